// stream.hpp -- pieces shared by the streaming matmul kernels (mmv.hip,
// mmqt.hip): LDS-writing buffer loads, raw barriers and wait immediates, a
// cheap uniform division, and the cursor that walks a workgroup's run of
// (tile, super-block) units in chunks.
#pragma once

#include "common.hpp"

#include <type_traits>
#include <utility>

namespace iq4xs {
namespace stream {

constexpr int BUFFER_FLAGS = 0x00020000;   // raw buffer resource, gfx9 family
constexpr uint32_t OOB = 0x80000000u;      // buffer offset past every range: loads return 0

constexpr int round_up_c(int x, int a) { return (x + a - 1) / a * a; }

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): LDS operations done and at most n vector memory
// operations of this wavefront outstanding; or LDS operations done only.
constexpr int wait_vm_lds(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
constexpr int WAIT_LDS = 15 | (3 << 14) | (7 << 4);

// LDS area I of SZ bytes of the calling kernel.
template <int I, int SZ>
__device__ __forceinline__ char *lds_area()
{
    __shared__ __attribute__((aligned(16))) char a[SZ];
    return a;
}

template <int... I, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F &&f)
{
    (f(std::integral_constant<int, I>()), ...);
}

// One 16-byte-per-lane buffer load that writes LDS: lane i's 16 bytes from
// rsrc at voffset land at lds_dst + 16*i (zeros when voffset is out of
// range).  Written as assembly so that the compiler neither waits for these
// loads by itself (it would make every LDS read wait for all of them, also
// for the loads into other buffers) nor moves memory operations across them;
// the kernel waits for them explicitly.  M0 holds the LDS address; the kernel
// uses M0 for nothing else.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, const char *lds_dst, uint32_t voffset)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voffset), "s"(rsrc)
                 : "memory", "m0");
}
// x / D for 0 <= x < LIM with one 24-bit multiply and a shift: the smallest
// shift S whose multiplier ceil(2^S / D) gives the exact quotient for every
// x < LIM, checked exhaustively at compile time.
struct DivMagic {
    uint32_t mul, shift;
};
template <uint32_t D, uint32_t LIM>
constexpr DivMagic div_magic()
{
    for (uint32_t s = 0; s < 32; s++) {
        const uint64_t mg = ((1ull << s) + D - 1) / D;
        if (mg >= (1u << 24) || mg * (LIM - 1) >= (1ull << 32))
            continue;
        bool ok = true;
        for (uint32_t x = 0; x < LIM && ok; x++)
            ok = (uint32_t)((x * mg) >> s) == x / D;
        if (ok)
            return DivMagic{(uint32_t)mg, s};
    }
    return DivMagic{0, 0};
}
template <uint32_t D, uint32_t LIM>
__device__ __forceinline__ uint32_t div_small(uint32_t x)
{
    constexpr DivMagic m = div_magic<D, LIM>();
    static_assert(m.mul != 0, "no 24-bit multiplier for this divisor and range");
    return (uint32_t)__umul24(x, m.mul) >> m.shift;
}

// Keeps the registers of v allocated, unchanged, up to this point (so that
// nothing else is written into a register the matrix core may still be
// writing, which would stall the wavefront).
typedef int v16i_keep __attribute__((ext_vector_type(16)));
__device__ __forceinline__ void keep_live(const v16i_keep &v)
{
    asm volatile("" ::"v"(v));
}
#pragma clang diagnostic pop

// v from the lane D lanes below in the same row of 16 lanes (0 for the first
// D lanes of the row).
template <int D>
__device__ __forceinline__ float shr_row(float v, std::integral_constant<int, D>)
{
    static_assert(D >= 1 && D <= 15, "row shift");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 | D, 0xF, 0xF, true));
}

// A barrier that neither waits for the loads in flight nor lets the compiler
// move memory operations across it (the caller waits for what it needs).
__device__ __forceinline__ void raw_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// A chunk: tile t, super-blocks j0..j0+cl-1 (cl = 0: past the run), flags
// bit 0 = the tile's units end with it, bit 1 = the tile belongs to this
// workgroup alone.
struct Chunk {
    int t, j0, cl, flags;
};

// Walks the run [ua, ub) of units in chunks (all values wavefront-uniform).
// Runs of units over at most MAXG workgroups, computed on the host: run g is
// units [u[g], u[g+1]) and starts in tile t[g].
constexpr int MAXG = 256;
struct Runs {
    int u[MAXG + 1];
    int t[MAXG];
};

struct Cursor {
    int u, t, j, ua, ub, nb;
    __device__ Chunk next(int ch)
    {
        Chunk c{t, j, 0, 0};
        if (u < ub) {
            int l = ub - u;
            l = l < nb - j ? l : nb - j;
            const int wl = (j & ~1) + ch - j;
            l = l < wl ? l : wl;
            const bool ends = j + l == nb || u + l == ub;
            const bool owned = t * nb >= ua && (t + 1) * nb <= ub;
            c.cl = l;
            c.flags = (ends ? 1 : 0) | (owned ? 2 : 0);
            u += l;
            j += l;
            if (j == nb) {
                j = 0;
                t++;
            }
        }
        return c;
    }
};

}  // namespace stream
}  // namespace iq4xs
