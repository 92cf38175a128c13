// ag_device.hpp -- device-side building blocks shared by the gfx950 kernels of libaggemm:
// bf16 vector types, buffer resources for LDS-DMA loads, and the chunk-flag protocol.
//
// Flag protocol (fused AllGather + MatMul article, "数据搬运与细粒度同步" and
// "wait_signal 的实现与语义"): a chunk's rows must be visible before its flag says so.  The
// copy stores its bytes write-through (they reach memory, none stays dirty in an XCD's L2) and
// drains them before it counts; counts and flags are read-modify-write atomics at the device's
// point of coherence, so a consumer on any of the eight XCDs (separate L2s) that sees a flag
// finds the chunk's bytes in memory.  A consumer's own caches hold no line of a chunk before its
// flag rises, unless rows are not whole cache lines; then it invalidates with an agent-scope
// acquire.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ag {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource word 3 for gfx9-family parts (raw buffer, 32-bit dword format).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                             kRsrcWord3);
}

// 16 bytes from global memory (rsrc + voffset) straight into LDS: lane l of the wave writes
// bytes [16 l, 16 l + 16) after the wave-uniform LDS address `lds_wave_base`.  An offset at or
// beyond the resource's size yields zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, void* lds_wave_base, uint32_t voffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_wave_base, 16, (int)voffset, 0, 0, 0);
}

// A value every lane of the workgroup holds (one lane wrote it to LDS before a barrier), made
// wave-uniform for the compiler.  Loop exits and branches around barriers must depend only on
// such values: a condition the compiler believes divergent gets structurized per lane, and a
// one-lane region inside a loop with barriers can then be moved out of the loop while the other
// lanes keep iterating.
__device__ __forceinline__ int64_t uniform_i64(int64_t v)
{
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt encodings (gfx9): vmcnt in [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// At most N vector memory operations of this wave still outstanding (N < 64).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0x0000); }

// Workgroup barrier after which every wave reads the LDS values any wave wrote before it.  The
// LDS writes are drained here explicitly (lgkmcnt 0, with a compiler memory barrier) instead of
// being left to the lowering of __syncthreads(), which was seen to drop that wait on a loop
// back edge: a wave could then pass the barrier and read the previous value.
__device__ __forceinline__ void barrier_after_lds_write()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
}

// ----------------------------------------------------------------------------------- flags
// Every access to a word that another workgroup writes is a read-modify-write atomic: the eight
// XCDs have separate L2s, and an RMW is resolved at the device's point of coherence, so a poll
// can never keep returning a copy cached in the polling XCD's L2.
//
// Each one is issued by lane 0 of the calling wave alone (an if-then with nothing inside but the
// atomic, result broadcast with readfirstlane): issued by all 64 lanes, an atomic becomes 64
// operations on one address, serialised at its memory channel.  Callers are whole waves in
// wave-uniform control flow.
__device__ __forceinline__ bool is_lane0() { return (threadIdx.x & 63) == 0; }

__device__ __forceinline__ uint32_t wave_fetch_add(uint32_t* p, uint32_t v)
{
    uint32_t r = 0;
    if (is_lane0())
        r = __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_amdgcn_readfirstlane(r);
}

__device__ __forceinline__ uint32_t wave_fetch_or(uint32_t* p, uint32_t v)
{
    uint32_t r = 0;
    if (is_lane0())
        r = __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_amdgcn_readfirstlane(r);
}

__device__ __forceinline__ void wave_exchange(uint32_t* p, uint32_t v)
{
    if (is_lane0())
        (void)__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wave_add_u64(uint64_t* p, uint64_t v)
{
    if (is_lane0())
        (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t flag_peek(uint32_t* f) { return wave_fetch_add(f, 0u); }

__device__ __forceinline__ void flag_publish(uint32_t* f, uint32_t value) { wave_exchange(f, value); }

__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Status word [code, chunk, tile, epoch]: the first failure since the host last read it wins the
// first three words (what ag_check reports); the fourth always takes the failing call's epoch, so
// the other waits of that call -- and only of that call -- give up at once.  Called by a whole wave.
__device__ __forceinline__ void report_failure(uint32_t* status, uint32_t code, uint32_t chunk, uint32_t tile,
                                               uint32_t epoch)
{
    if (wave_fetch_or(&status[0], code) == 0) {
        wave_exchange(&status[1], chunk);
        wave_exchange(&status[2], tile);
    }
    wave_exchange(&status[3], epoch);
}

}  // namespace ag
