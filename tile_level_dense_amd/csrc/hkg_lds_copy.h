// Buffer -> LDS copies (buffer_load_dwordx4 ... lds) issued as inline asm,
// shared by the tile and skinny kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hkg {
namespace dma {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// The 128-bit buffer descriptor of __builtin_amdgcn_make_buffer_rsrc(p, 0,
// bytes, 0x00020000), as four dwords (base, base high bits with stride 0,
// range, word 3: raw buffer of 32-bit data, out-of-range offsets read zero).
__device__ __forceinline__ i32x4 rsrc_words(const void* p, int bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)p;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), bytes, 0x00020000};
}

// One buffer -> LDS copy of 16 bytes per lane: lane i's bytes at offset voff
// of the buffer land at LDS address lds + 16 i (lds must be wave-uniform).
// Written as inline asm so that the compiler does not order later LDS reads
// after it: for the builtin it waits for every copy in flight (vmcnt(0))
// before each LDS read it cannot prove disjoint, which leaves no copy in
// flight across a K step.  The compiler does not count these copies in its
// own vmcnt waits; callers wait for them explicitly, and the compiler's waits
// for its own loads only become stricter by the copies issued after them.
// M0 holds the LDS address; one wait state separates its write from the
// copy.  M0 is named as clobbered, so the compiler re-establishes it before
// any later use of its own (the buffer->LDS builtin and LDS-direct forms
// also take their LDS address from M0).
// (clang notes that M0 is a reserved register; the clobber still marks the
// asm statement as defining it, which is what later M0 users need.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy_to_lds(i32x4 rsrc, const char* lds, uint32_t voff)
{
    const uint32_t m0 = (uint32_t)(size_t)(lds_void*)lds;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace dma
}  // namespace hkg
