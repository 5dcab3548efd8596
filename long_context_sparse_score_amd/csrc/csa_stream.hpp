// csa_stream.hpp -- streaming packed rows through a per-wave LDS ring with
// direct-to-LDS loads.
//
// A chunk is 64 consecutive 68-byte rows (4352 bytes): four coalesced
// 1024-byte global_load_lds_dwordx4 (one 16-byte piece per lane) plus a
// 256-byte tail by lanes 0..15.  The rows land in LDS exactly as stored, and
// each lane then reads its matrix-core operand (16 code bytes and the scale
// byte of row l%16, block l/16) with ordinary LDS loads.
//
// The loads are issued from inline assembly on purpose: the compiler then
// does not see LDS writes in flight, so it neither forces a full drain of
// the load counter before every LDS access nor reorders around them; the
// consumer waits explicitly (wait_vmcnt) for exactly the chunk it is about to
// read.  Any wait the compiler inserts for its own loads stays correct,
// because additional outstanding loads only make such waits longer.  No code
// between a chunk's issue and its wait may issue other vector memory
// instructions, or the explicit count would be off.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa_device.hpp"

namespace csa {

constexpr int kChunkRows = 64;
constexpr int kChunkBytes = kChunkRows * kIdxRowBytes;  // 4352
constexpr int kChunkDma = 5;                             // load instructions per chunk
constexpr int kChunkSlot = kChunkBytes + 64;             // LDS bytes per ring slot (16-aligned)

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per active lane from `g` to LDS address lds + 16 * lane (M0 = lds).
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
// 16 bytes per active lane from the wave-uniform base `sbase` plus the lane's
// byte offset `voff` to LDS address lds + 16 * lane (M0 = lds); the scalar
// base keeps the per-chunk address arithmetic off the vector ALU.
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
// 4 bytes per active lane from `g` to LDS address lds + 4 * lane (M0 = lds).
__device__ __forceinline__ void dma4(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
// 4 bytes per active lane from sbase + voff (sbase wave-uniform) to LDS
// address lds + 4 * lane (M0 = lds).
__device__ __forceinline__ void dma4s(const void *sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector memory instructions are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until this wave's LDS loads and stores have completed.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// A wave-uniform pointer moved to scalar registers (readfirstlane works on
// 32 bits: each half separately).
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t *>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// Lane offsets of the five 16-byte pieces of a chunk: 16 lane + 1024 i.
struct ChunkLanes {
  uint32_t off[kChunkDma];
};
__device__ __forceinline__ ChunkLanes chunk_lanes(int lane) {
  ChunkLanes c;
#pragma unroll
  for (int i = 0; i < kChunkDma; ++i) c.off[i] = 16u * (uint32_t)lane + 1024u * (uint32_t)i;
  return c;
}

// Issue the loads of the chunk whose first row starts at the wave-uniform
// address `chunk` into the LDS slot `slot` (wave-uniform); same pieces and
// alignment rules as issue_chunk.
__device__ __forceinline__ void issue_chunk_s(const uint8_t *chunk, const ChunkLanes &cl, uint32_t slot, int lane) {
  slot = __builtin_amdgcn_readfirstlane(slot);
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16s(chunk, cl.off[i], slot + 1024 * i);
  if (lane < 16) dma16s(chunk, cl.off[4], slot + 4096);
}

// Issue the loads of the chunk of rows [r0, r0 + 64) into the LDS slot at
// `slot` (wave-uniform).  The whole chunk must lie inside the buffer, and the
// buffer must start 16-byte aligned (64 rows are 4352 = 272 * 16 bytes, so
// every piece is then an aligned 16 bytes).
__device__ __forceinline__ void issue_chunk(const uint8_t *__restrict__ rows, int64_t r0, uint32_t slot, int lane) {
  const uint8_t *g = rows + r0 * kIdxRowBytes;
  slot = __builtin_amdgcn_readfirstlane(slot);
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16(g + 1024 * i + 16 * lane, slot + 1024 * i);
  if (lane < 16) dma16(g + 4096 + 16 * lane, slot + 4096);
}

}  // namespace csa
