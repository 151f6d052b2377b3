// Store-burst probe: the local-memory form of the periodic and isolated
// burst microbenchmarks of X-Stage, Section 3.1 ("Remote-Store
// Microbenchmarks"), whose timings calibrate the Burst–Gap parameters
// (T_iss^0, R, Q) of Section 3.2-3.5 for stores a CU issues into its own HBM.
//
// K producers (one wavefront each, one workgroup each) start together and
// repeat: read the clock, issue a burst of B bytes of 16-byte vector stores
// (64 lanes x 16 B per instruction, consecutive 1 KiB blocks), read the clock
// again once the last store has issued (the sender-visible issue time: a
// store's issue stalls only under backpressure, its completion is not
// awaited), then idle for the producer-side gap G with no memory traffic.
// Each producer writes its own ring of the buffer, so consecutive bursts reach
// new lines until the ring wraps.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kStartSpin = 1 << 14;     // bounded wait for the common start time
constexpr uint64_t kStartLead = 2000;   // clock ticks (20 us at 100 MHz) from producer 0's reading to the start

__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }

__global__ __launch_bounds__(64) void store_burst_kernel(uint8_t* __restrict__ buf, size_t ring, int B, int reps,
                                                         uint64_t gap, uint64_t* __restrict__ rec,
                                                         uint64_t* __restrict__ epoch) {
  const int k = blockIdx.x, lane = threadIdx.x;
  uint8_t* base = buf + (size_t)k * ring;
  // common start: producer 0 publishes a time a few microseconds ahead, the
  // others wait for it (a bounded wait: without it they start at once)
  // The epoch is exchanged with device-scope atomic read-modify-writes (the
  // same coherence path as the expert GEMM's readiness counters), and
  // whatever value is read, the wait is capped at 2 kStartLead ticks from
  // this producer's own clock: no value in memory can hold a producer back.
  const uint64_t mine = now();
  uint64_t t0 = mine + kStartLead;
  if (k == 0) {
    if (lane == 0) __hip_atomic_fetch_max(epoch, t0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    uint64_t v = 0, zero = 0;
    asm volatile("" : "+v"(zero));  // an addend the compiler cannot fold: a true read-modify-write
    for (int spins = 0; spins < kStartSpin; ++spins) {
      v = __hip_atomic_fetch_add(epoch, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v) break;
      __builtin_amdgcn_s_sleep(1);
    }
    t0 = v ? v : mine;
  }
  t0 = __builtin_amdgcn_readfirstlane((uint32_t)t0) | ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(t0 >> 32)) << 32);
  if (t0 > mine + 2 * kStartLead) t0 = mine + 2 * kStartLead;
  while (now() < t0) __builtin_amdgcn_s_sleep(1);  // ends within 2 kStartLead ticks

  const int per = B >> 10;  // store instructions per burst
  size_t off = 0;
  for (int r = 0; r < reps; ++r) {
    asm volatile("" ::: "memory");
    const uint64_t ts = now();
    asm volatile("" ::: "memory");
    uint4* dst = reinterpret_cast<uint4*>(base + off) + lane;
    for (int i = 0; i < per; ++i) dst[(size_t)i * 64] = make_uint4((uint32_t)r, (uint32_t)i, (uint32_t)k, (uint32_t)lane);
    asm volatile("" ::: "memory");
    const uint64_t ti = now();
    asm volatile("" ::: "memory");
    if (lane == 0) {
      rec[((size_t)k * reps + r) * 2] = ts;
      rec[((size_t)k * reps + r) * 2 + 1] = ti;
    }
    off += (size_t)B;
    if (off + (size_t)B > ring) off = 0;
    while (now() - ti < gap) __builtin_amdgcn_s_sleep(1);  // the gap: no memory traffic
  }
}

__global__ void zero_u64_kernel(uint64_t* p) { *p = 0; }

}  // namespace

hipError_t launch_store_burst(int K, int B, int reps, double gap_us, void* buf, size_t buf_bytes, uint64_t* rec,
                              hipStream_t s) {
  const size_t ring = (buf_bytes / (size_t)K) & ~(size_t)1023;
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return e;
  if (khz <= 0) return hipErrorInvalidValue;
  const uint64_t gap = (uint64_t)(gap_us * khz * 1e-3 + 0.5);  // clock ticks
  uint64_t* epoch = rec + (size_t)K * reps * 2;
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, s, epoch);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(store_burst_kernel, dim3(K), dim3(64), 0, s, static_cast<uint8_t*>(buf), ring, B, reps, gap,
                     rec, epoch);
  return hipGetLastError();
}

}  // namespace moe
