// Pieces shared by the 4-bit head-dim-256 attention kernels on gfx950: the
// stage layout of the direct-to-LDS copies, the fp16 dequantisation of a code
// word, the matrix instructions with their hazard padding and the O
// accumulators pinned to the accumulation registers.
#pragma once

#include <type_traits>

#include "attn_sched.h"

namespace sv {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int D = 256;
constexpr int T = 128;                      // positions per DMA stage
constexpr int CROW = D / 2;                 // code bytes per row
constexpr int SROW = D / 16;                // scale bytes per row
constexpr int STAGE = 2 * T * (CROW + SROW);
constexpr int NKB = STAGE / 1024;           // 1 KB DMA instructions per stage
constexpr int KCI = T * CROW / 1024, KSI = T * SROW / 1024;
constexpr int CPS = T / 32;                 // 32-position chunks per stage
constexpr int FROW = D * 2;                 // fp16 staging row bytes
constexpr int FST = 32 * FROW;              // one staged chunk of K or V
constexpr int PROW = 80;                    // P row bytes (32 fp16 + 16 padding)
constexpr int kMaxPages = 512;
static_assert(KCI * 1024 == T * CROW && KSI * 1024 == T * SROW, "stage layout");

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void dma16(uint32_t lds_base, const void *gptr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(gptr)
                 : "memory", "m0");
}

__device__ __forceinline__ void dma16s(uint32_t lds_base, const void *sbase, uint32_t voff) {
    const uint64_t a = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(u)
                 : "memory", "m0");
}

// (w & m) | c in one instruction
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "v"(m), "v"(c));
    return r;
}

// Eight 4-bit codes (one 32-bit word, value 2t in the low nibble of byte t)
// times the block scale s (both halves), as fp16 in the order
// (0, 4, 2, 6, 1, 5, 3, 7).
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, h2 s, uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
    const h2 off = {(_Float16)-1032.f, (_Float16)-1032.f};   // 1024 + n -> n - 8
    const h2 sx = {(_Float16)0.0625f, (_Float16)0.0625f};     // (1024 + 16 n) / 16 - 72 -> n - 8
    const h2 o2 = {(_Float16)-72.f, (_Float16)-72.f};
    const uint32_t w8 = w >> 8;
    const h2 a = __builtin_bit_cast(h2, and_or(w, m_lo, magic));     // values 0, 4
    const h2 b = __builtin_bit_cast(h2, and_or(w, m_hi, magic));     // values 1, 5
    const h2 c = __builtin_bit_cast(h2, and_or(w8, m_lo, magic));    // values 2, 6
    const h2 d = __builtin_bit_cast(h2, and_or(w8, m_hi, magic));    // values 3, 7
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, (a + off) * s);
    r[1] = __builtin_bit_cast(uint32_t, (c + off) * s);
    r[2] = __builtin_bit_cast(uint32_t, (b * sx + o2) * s);
    r[3] = __builtin_bit_cast(uint32_t, (d * sx + o2) * s);
    return r;
}

// ---- matrix instructions ------------------------------------------------------
// S^T = K Q^T runs with its accumulators in architectural VGPRs.  The O^T
// accumulators (up to 24 tiles of 16 x 16 fp32) live in the accumulation
// registers a0..a95 for the whole kernel: tile I in a[4I .. 4I+3], written
// and read only by the inline assembly below (the kernel is compiled in the
// VGPR matrix form and never spills, so the compiler itself uses no
// accumulation register; the clobbers make it count them in the kernel's
// register total).  With the compiler's own allocation the O tiles moved to
// other registers inside the loop and were copied back on every chunk.
// Hazards the compiler cannot see are covered here: s_nop 1 before an S
// instruction (its operands may have just been written by vector code),
// mfma_drain() / mfma_drain_s() before vector code reads a matrix result.
__device__ __forceinline__ f32x4 mfma_s_first(h8 a, h8 b) {
    f32x4 d;
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ void mfma_s_acc(f32x4 &c, h8 a, h8 b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

template <int I> struct OTile;
#define SV_OTILE(I, R0, R1, R2, R3)                                                                        \
    template <> struct OTile<I> {                                                                          \
        static __device__ __forceinline__ void zero() {                                                    \
            asm volatile("v_accvgpr_write_b32 a" #R0 ", 0\n\tv_accvgpr_write_b32 a" #R1                     \
                         ", 0\n\tv_accvgpr_write_b32 a" #R2 ", 0\n\tv_accvgpr_write_b32 a" #R3 ", 0" ::       \
                             : "a" #R0, "a" #R1, "a" #R2, "a" #R3);                                         \
        }                                                                                                  \
        static __device__ __forceinline__ void mac(h8 a, h8 b) {                                           \
            asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 a[" #R0 ":" #R3 "], %0, %1, a[" #R0 ":" #R3 "]"  \
                         ::"v"(a), "v"(b)                                                                  \
                         : "a" #R0, "a" #R1, "a" #R2, "a" #R3);                                             \
        }                                                                                                  \
        static __device__ __forceinline__ f32x4 read() {                                                   \
            f32x4 r;                                                                                       \
            asm volatile("v_accvgpr_read_b32 %0, a" #R0 "\n\tv_accvgpr_read_b32 %1, a" #R1                  \
                         "\n\tv_accvgpr_read_b32 %2, a" #R2 "\n\tv_accvgpr_read_b32 %3, a" #R3                \
                         : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]));                                 \
            return r;                                                                                      \
        }                                                                                                  \
        static __device__ __forceinline__ void scale(float f) {                                            \
            float t0, t1, t2, t3;                                                                          \
            asm volatile("v_accvgpr_read_b32 %0, a" #R0 "\n\tv_accvgpr_read_b32 %1, a" #R1                  \
                         "\n\tv_accvgpr_read_b32 %2, a" #R2 "\n\tv_accvgpr_read_b32 %3, a" #R3                \
                         "\n\tv_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4"            \
                         "\n\tv_mul_f32 %3, %3, %4"                                                        \
                         "\n\tv_accvgpr_write_b32 a" #R0 ", %0\n\tv_accvgpr_write_b32 a" #R1 ", %1"           \
                         "\n\tv_accvgpr_write_b32 a" #R2 ", %2\n\tv_accvgpr_write_b32 a" #R3 ", %3"           \
                         : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)                                       \
                         : "v"(f)                                                                          \
                         : "a" #R0, "a" #R1, "a" #R2, "a" #R3);                                             \
        }                                                                                                  \
    };
SV_OTILE(0, 0, 1, 2, 3)
SV_OTILE(1, 4, 5, 6, 7)
SV_OTILE(2, 8, 9, 10, 11)
SV_OTILE(3, 12, 13, 14, 15)
SV_OTILE(4, 16, 17, 18, 19)
SV_OTILE(5, 20, 21, 22, 23)
SV_OTILE(6, 24, 25, 26, 27)
SV_OTILE(7, 28, 29, 30, 31)
SV_OTILE(8, 32, 33, 34, 35)
SV_OTILE(9, 36, 37, 38, 39)
SV_OTILE(10, 40, 41, 42, 43)
SV_OTILE(11, 44, 45, 46, 47)
SV_OTILE(12, 48, 49, 50, 51)
SV_OTILE(13, 52, 53, 54, 55)
SV_OTILE(14, 56, 57, 58, 59)
SV_OTILE(15, 60, 61, 62, 63)
SV_OTILE(16, 64, 65, 66, 67)
SV_OTILE(17, 68, 69, 70, 71)
SV_OTILE(18, 72, 73, 74, 75)
SV_OTILE(19, 76, 77, 78, 79)
SV_OTILE(20, 80, 81, 82, 83)
SV_OTILE(21, 84, 85, 86, 87)
SV_OTILE(22, 88, 89, 90, 91)
SV_OTILE(23, 92, 93, 94, 95)
#undef SV_OTILE

// f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// The same wait tied to the score tiles the last matrix instructions wrote:
// the compiler sees the hazard padding as the producer of the tiles, so no
// vector instruction reading them can be scheduled above it (the padding of
// mfma_drain orders only memory and other volatile statements).
template <int N>
__device__ __forceinline__ void mfma_drain_s(f32x4 (&s)[N]) {
    static_assert(N >= 1 && N <= 3, "one to three score tiles");
    if constexpr (N == 1) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0])::"memory");
    } else if constexpr (N == 2) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1])::"memory");
    } else {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2])::"memory");
    }
}

}  // namespace
}  // namespace sv
