// Per-wave LDS ring fed by asynchronous global->LDS loads (gfx950
// global_load_lds_dwordx4): a wave keeps the key/value rows of its next
// tiles in flight without holding them in registers.
//
// A slot holds one tile of 16 key rows and 16 value rows (head_dim 128,
// bf16): [K 4 KB][V 4 KB].  Inside each 4 KB half, 16-byte chunk s holds
// row t = s >> 4, column chunk u = (s & 15) ^ t; the XOR swizzle makes the
// 16-byte operand reads of both the MFMA path and the draft path free of
// LDS bank conflicts.
//
// The loads (and the logit stores that are interleaved with them) are
// issued from inline asm and consumed after an explicit vmcnt wait, so the
// number of memory operations between a tile's issue and its use is known
// exactly; the compiler would otherwise drain every outstanding load before
// each LDS read of the ring.  Vector memory operations of a wave complete in
// issue order, so waiting until at most N are outstanding guarantees that
// everything issued before the last N has landed.
#pragma once

#include "sspec_common.hpp"

namespace sspec {

constexpr int kSlotBytes = 8192;
constexpr int kRing = 3;  // slots per wave by default: two tiles in flight while one is used

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Each helper below sets M0 and issues its loads in ONE asm statement (M0 is
// declared clobbered, so the compiler keeps none of its own values there
// across it), with the wait states the hardware requires written out,
// because the compiler's hazard handling cannot see into inline asm:
//   * an SALU write of M0 needs 1 wait state before an LDS-DMA load reads it
//     (otherwise the load uses the previous M0 and lands in the wrong place);
//   * an SGPR written by a VALU op (v_readfirstlane) needs 5 wait states
//     before a vector memory instruction reads it as its base address.
// 64 lanes x 16 B per load: lane l's chunk lands at LDS m0 + imm + 16*l; the
// immediate offset is added to the global address as well.

// 4 loads into LDS [lds, lds + 4 KB): load c reads sbase + voff[c] + 1024*c
// (sbase wave-uniform).  4 vector memory operations.  The key/value stream is
// read once per launch, so the loads carry the non-temporal hint (nt): they
// then do not push the logit dump, re-read soon after, out of the caches.
__device__ __forceinline__ void dma_4k_s(uint32_t lds, const void* sbase, const uint32_t (&voff)[4]) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %1, %5 offset:0 nt\n\t"
      "global_load_lds_dwordx4 %2, %5 offset:1024 nt\n\t"
      "global_load_lds_dwordx4 %3, %5 offset:2048 nt\n\t"
      "global_load_lds_dwordx4 %4, %5 offset:3072 nt"
      ::"s"(lds), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(sbase)
      : "memory", "m0");
}
// same with per-lane 64-bit addresses: load c reads a[c] + 1024*c.
__device__ __forceinline__ void dma_4k_v(uint32_t lds, const void* a0, const void* a1, const void* a2,
                                         const void* a3) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off offset:0 nt\n\t"
      "global_load_lds_dwordx4 %2, off offset:1024 nt\n\t"
      "global_load_lds_dwordx4 %3, off offset:2048 nt\n\t"
      "global_load_lds_dwordx4 %4, off offset:3072 nt"
      ::"s"(lds), "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory", "m0");
}
// Wait until the wave's LDS reads have returned: a slot is refilled only
// after the reads of its previous tile are done.
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most n vector memory operations are outstanding (n <= 47;
// larger n waits for all)
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (n) {
#define SSPEC_W(i) case i: wait_vm<i>(); break;
    SSPEC_W(0) SSPEC_W(1) SSPEC_W(2) SSPEC_W(3) SSPEC_W(4) SSPEC_W(5) SSPEC_W(6) SSPEC_W(7)
    SSPEC_W(8) SSPEC_W(9) SSPEC_W(10) SSPEC_W(11) SSPEC_W(12) SSPEC_W(13) SSPEC_W(14) SSPEC_W(15)
    SSPEC_W(16) SSPEC_W(17) SSPEC_W(18) SSPEC_W(19) SSPEC_W(20) SSPEC_W(21) SSPEC_W(22) SSPEC_W(23)
    SSPEC_W(24) SSPEC_W(25) SSPEC_W(26) SSPEC_W(27) SSPEC_W(28) SSPEC_W(29) SSPEC_W(30) SSPEC_W(31)
    SSPEC_W(32) SSPEC_W(33) SSPEC_W(34) SSPEC_W(35) SSPEC_W(36) SSPEC_W(37) SSPEC_W(38) SSPEC_W(39)
    SSPEC_W(40) SSPEC_W(41) SSPEC_W(42) SSPEC_W(43) SSPEC_W(44) SSPEC_W(45) SSPEC_W(46) SSPEC_W(47)
#undef SSPEC_W
    default: wait_vm<0>(); break;
  }
}

// Byte offset, inside a 4 KB tile half, of (row t, 16-byte column chunk u).
__device__ __forceinline__ uint32_t ring_chunk(int t, int u) { return (uint32_t)(t * 16 + (u ^ t)) * 16u; }

// Global byte offset (within a 4 KB page of 16 rows) that lane l must fetch
// for load instruction c (0..3) so that the chunk lands at its swizzled
// place: LDS chunk 64*c + l is row t = 4*c + l/16, column (l & 15) ^ t.  The
// instruction's immediate offset adds 1024*c to both sides, so this is the
// remainder.
__device__ __forceinline__ uint32_t ring_src_off(int c, int lane) {
  const int t = 4 * c + (lane >> 4);
  return (uint32_t)((lane >> 4) * 256 + (((lane & 15) ^ t) * 16));
}

// Issue one page (16 consecutive rows of one KV head, 4 KB of K and 4 KB of
// V) into slot `slot_lds`: 8 vector memory operations.
__device__ __forceinline__ void ring_issue_page(uint32_t slot_lds, const uint16_t* kpage, const uint16_t* vpage,
                                                const uint32_t (&soff)[4]) {
  kpage = wave_uniform(kpage);
  vpage = wave_uniform(vpage);
  slot_lds = __builtin_amdgcn_readfirstlane(slot_lds);
  dma_4k_s(slot_lds, kpage, soff);
  dma_4k_s(slot_lds + 4096, vpage, soff);
}

// Issue 16 gathered rows (row ids of the pool, 256 B each) into a slot:
// lane l of load c fetches row t = 4c + l/16, chunk (l & 15) ^ t.
// 8 vector memory operations.
__device__ __forceinline__ void ring_issue_rows(uint32_t slot_lds, const uint16_t* kp, const uint16_t* vp,
                                                const uint32_t (&rows)[4], int lane) {
  slot_lds = __builtin_amdgcn_readfirstlane(slot_lds);
  const char* ka[4];
  const char* va[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = 4 * c + (lane >> 4);
    // minus 1024*c: the load's immediate offset adds it back
    const size_t off = (size_t)rows[c] * (kD * 2) + (size_t)(((lane & 15) ^ t) * 16) - (size_t)(1024 * c);
    ka[c] = reinterpret_cast<const char*>(kp) + off;
    va[c] = reinterpret_cast<const char*>(vp) + off;
  }
  dma_4k_v(slot_lds, ka[0], ka[1], ka[2], ka[3]);
  dma_4k_v(slot_lds + 4096, va[0], va[1], va[2], va[3]);
}

}  // namespace sspec
