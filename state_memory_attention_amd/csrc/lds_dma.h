// Device helpers shared by the MFMA kernels: direct global->LDS loads, explicit
// s_waitcnt immediates and the swizzled layout of a staged chunk memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dart {

// Cache-policy bit of a buffer access for data streamed once: non-temporal,
// so that the stream does not evict data that other blocks re-read from L2.
constexpr int kNonTemporal = 2;

// A pointer made wave-uniform in the compiler's eyes (its value is the same
// in every lane): a buffer resource formed from it then lives in scalar
// registers, where a resource the compiler takes for divergent costs a loop
// over lanes around every access.
template <typename T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// Block order of the token-tile kernels (a block = one 128-token tile of one
// (b, h); head slots padded to a multiple of 8).  Consecutive block numbers
// go round-robin to the 8 XCDs, so head slot xcd + 8 k always lands on XCD
// xcd; each XCD takes its heads one after another and every head's tiles
// last first (longest history first).  The tiles in flight on an XCD then
// share one or two heads' chunk memories, which stay in its L2 (with heads
// interleaved, the working set of every head of the XCD exceeded it).
struct TileItem {
  int bh, tile;
};
__device__ __forceinline__ TileItem head_major_tile(int blk, int n_tiles) {
  const int xi = blk >> 3;
  return TileItem{(blk & 7) + 8 * (xi / n_tiles), n_tiles - 1 - xi % n_tiles};
}

// One direct global->LDS load: every lane fetches 16 bytes from `src`, and
// lane l's bytes land at lds + 16 l (the LDS address is wave-uniform).
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// The same through a buffer resource covering bytes [0, nbytes) of `base`
// (a lane offset past the end reads zeros).  The compiler counts a
// global->LDS load as possibly outstanding on the LDS counter as well, which
// turns every LDS wait it places while one is in flight into a full drain;
// the buffer form is counted on the vector-memory counter only, so loads that
// stay in flight across a loop use it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t nbytes) {
  // word 3: 32-bit data format, the value every gfx9 raw buffer access uses
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                           0, 0, 0);
}
// The same with the non-temporal policy, for operands that no other block
// reads again (a stream read once sustains more bandwidth this way).
__device__ __forceinline__ void buf_dma16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                           0, 0, kNonTemporal);
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt
// in 11:8; a field at its maximum does not wait).  Issued as builtins, not as
// inline asm, so that the compiler's own wait insertion takes them into account.
constexpr unsigned kWaitAll = 0x0000;
constexpr unsigned kWaitVm0 = 0x0f70;
constexpr unsigned kWaitLgkm0 = 0xc07f;
constexpr unsigned kWaitVm4Lgkm0 = 0x0074;
constexpr unsigned kWaitVm8Lgkm0 = 0x0078;

// Byte offset of 16-byte piece `piece` (0..15) of row `row` of a staged
// chunk memory dH_j^T (64 rows p of 128 bf16 n): 256-byte rows, pieces
// XOR-swizzled by the row so that MFMA operand reads of 16 bytes per lane are
// bank-conflict free.
__device__ __forceinline__ uint32_t mem_off(int row, int piece) {
  return (uint32_t)(row * 256 + ((piece ^ (row & 15)) << 4));
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Sum of a value over lanes l and l ^ 32 (the two half-waves).
__device__ __forceinline__ float halves_sum(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

}  // namespace dart
