// stream_ceiling.hip — the streaming-bandwidth probe declared in
// include/hlwq_stream.h: pure data movement in the access pattern of the HLWQ
// kernels (1 KB-contiguous direct-to-LDS loads, 1 KB-contiguous stores from
// LDS, streaming cache policy), at a caller-chosen read:write mix, used by
// bench.py as the practical HBM ceiling of a kernel's own traffic.
//
// Buffer resources span exactly one unit, so a lane whose 16-byte chunk lies
// past the unit's end is out of the resource's range: its load returns zeros
// without touching memory and its store is dropped.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "hlwq_stream.h"

namespace {

constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kNt = 2;         // streaming (nontemporal) cache policy

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t unit_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)p));
}

// wait until at most n (0..32) vector-memory operations of this wave are
// outstanding; they complete in issue order, so everything issued before the
// last n has completed
__device__ __forceinline__ void wait_vmcnt_le(uint32_t n) {
  switch (n) {
#define HLWQ_WAIT_CASE(k) \
  case k:                 \
    asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); \
    break;
    HLWQ_WAIT_CASE(1) HLWQ_WAIT_CASE(2) HLWQ_WAIT_CASE(3) HLWQ_WAIT_CASE(4) HLWQ_WAIT_CASE(5) HLWQ_WAIT_CASE(6)
    HLWQ_WAIT_CASE(7) HLWQ_WAIT_CASE(8) HLWQ_WAIT_CASE(9) HLWQ_WAIT_CASE(10) HLWQ_WAIT_CASE(11)
    HLWQ_WAIT_CASE(12) HLWQ_WAIT_CASE(13) HLWQ_WAIT_CASE(14) HLWQ_WAIT_CASE(15) HLWQ_WAIT_CASE(16)
#undef HLWQ_WAIT_CASE
    default:
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

__device__ __forceinline__ void load_unit(const uint8_t* src, uint32_t bytes, uint32_t ri, uint8_t* buf, int lane) {
  const auto r = unit_rsrc(src, bytes);
  for (uint32_t i = 0; i < ri; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(buf + 1024 * i), 16,
                                             1024u * i + 16u * lane, 0, 0, kNt);
}

// stores read the staging buffer cyclically (its content is irrelevant)
__device__ __forceinline__ void store_unit(uint8_t* dst, uint32_t bytes, uint32_t wi, uint32_t buf, uint32_t buf_bytes,
                                           int lane) {
  const auto w = unit_rsrc(dst, bytes);
  uint32_t o = 0;
  for (uint32_t i = 0; i < wi; ++i) {
    const u32x4 v = *(const lds_u32x4*)static_cast<uintptr_t>(buf + o + 16u * lane);
    __builtin_amdgcn_raw_buffer_store_b128(v, w, 1024u * i + 16u * lane, 0, kNt);
    o = (o + 1024u < buf_bytes) ? o + 1024u : 0u;
  }
}

// STG: LDS bytes per wave; PIPE: two buffers of STG / 2, the next unit's loads
// issued before this unit is waited for
template <int STG, bool PIPE>
__global__ void __launch_bounds__(kThreads) stream_mix_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                                uint32_t rb, uint32_t wb, uint32_t units) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[4 * STG];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* stage = lds + wave * STG;
  constexpr uint32_t kBuf = PIPE ? STG / 2 : STG;
  const uint32_t ri = (rb + 1023u) / 1024u, wi = (wb + 1023u) / 1024u;
  const uint32_t step = gridDim.x * 4u;
  uint32_t b = blockIdx.x * 4u + wave;
  if constexpr (!PIPE) {
    for (; b < units; b += step) {
      load_unit(src + static_cast<size_t>(b) * rb, rb, ri, stage, lane);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      store_unit(dst + static_cast<size_t>(b) * wb, wb, wi, lds_addr(stage), kBuf, lane);
      asm volatile("" ::: "memory");
    }
  } else {
    uint32_t cur = 0;
    if (b < units) load_unit(src + static_cast<size_t>(b) * rb, rb, ri, stage, lane);
    for (; b < units; b += step) {
      const uint32_t nb = b + step;
      if (nb < units) {
        load_unit(src + static_cast<size_t>(nb) * rb, rb, ri, stage + (cur ^ kBuf), lane);
        wait_vmcnt_le(ri);
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      store_unit(dst + static_cast<size_t>(b) * wb, wb, wi, lds_addr(stage + cur), kBuf, lane);
      asm volatile("" ::: "memory");
      cur ^= kBuf;
    }
  }
}

int compute_units() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int n = dev < 64 ? cus[dev].load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < 64) cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

extern "C" int hlwq_stream_mix(const void* src, void* dst, uint32_t read_bytes, uint32_t write_bytes, uint32_t units,
                               int variant, int workgroups_per_cu, void* hip_stream) {
  static const uint32_t kMaxRead[4] = {16384, 32768, 16384, 4096};
  if (variant < 0 || variant > 3 || workgroups_per_cu < 1 || workgroups_per_cu > 4) return -3;
  if (read_bytes % 16 || write_bytes % 16 || write_bytes == 0 || write_bytes > 32768 ||
      read_bytes > kMaxRead[variant])
    return -2;
  if (units == 0) return 0;
  if (!src || !dst) return -1;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u)) return -6;
  const dim3 grid(static_cast<uint32_t>(compute_units() * workgroups_per_cu)), block(kThreads);
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const uint8_t* in = static_cast<const uint8_t*>(src);
  uint8_t* out = static_cast<uint8_t*>(dst);
  using Kernel = void (*)(const uint8_t*, uint8_t*, uint32_t, uint32_t, uint32_t);
  static const Kernel kernels[4] = {stream_mix_kernel<16384, false>, stream_mix_kernel<32768, false>,
                                    stream_mix_kernel<32768, true>, stream_mix_kernel<8192, true>};
  uint32_t rb = read_bytes, wb = write_bytes, n = units;
  void* params[] = {&in, &out, &rb, &wb, &n};
  // the status of this launch itself, not an error an earlier call left pending
  return hipLaunchKernel(reinterpret_cast<const void*>(kernels[variant]), grid, block, params, 0, s) == hipSuccess
             ? 0
             : -5;
}
