// timeline.hpp -- per-wave timeline hooks for the FP8 row and table kernels.
//
// Measurement only.  Built with ALNP_TIMELINE (libalnp_timeline.so, never
// the product library), each wave of k_adaln_fp8_rows and
// k_adaln_fp8_table_lds reads the 100 MHz constant clock (s_memrealtime) at
// fixed points of its work and writes one record of eight 64-bit words to
// the buffer set by alnp_timeline_set:
//   [0] start            [1] x loads issued   [2] x landed (row sum formed)
//   [3] rstd known       [4] stores issued    [5] stores done (vmcnt 0)
//   [6] XCC_ID register  [7] HW_ID register (CU, SIMD and wave slot)
// Record (row * waves per row + wave) of a buffer of rows * 8 waves * 8
// words.  Without ALNP_TIMELINE every hook expands to nothing.
#pragma once

#ifdef ALNP_TIMELINE

namespace alnp {
// Set by alnp_timeline_set (producers.hip); null: no records.
extern __device__ unsigned long long* timeline_buf;
__device__ __forceinline__ unsigned long long timeline_now() { return __builtin_amdgcn_s_memrealtime(); }
}  // namespace alnp

// The clock reads of one wave, in a register array declared by ALNP_TL_VARS.
#define ALNP_TL_VARS unsigned long long tl_[5] = {0, 0, 0, 0, 0}
#define ALNP_TL_MARK(k) tl_[k] = alnp::timeline_now()
// A clock read that follows the computation of `value` (an empty asm that
// takes it as a register operand orders the read after it).
#define ALNP_TL_MARK_AFTER(k, value)                                                \
    do {                                                                            \
        asm volatile("" ::"v"(value));                                              \
        tl_[k] = alnp::timeline_now();                                              \
    } while (0)
// The stores-done read, then the record from lane 0 of each wave.
#define ALNP_TL_RECORD(row, waves)                                                  \
    do {                                                                            \
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                            \
        const unsigned long long t5_ = alnp::timeline_now();                        \
        unsigned long long* g_ = alnp::timeline_buf;                                \
        if (g_ && (threadIdx.x & 63) == 0) {                                        \
            unsigned long long* p_ =                                                \
                g_ + ((int64_t)(row) * (waves) + ((threadIdx.x >> 6) % (waves))) * 8; \
            for (int k_ = 0; k_ < 5; ++k_)                                          \
                p_[k_] = tl_[k_];                                                   \
            p_[5] = t5_;                                                            \
            p_[6] = __builtin_amdgcn_s_getreg(20 | (31 << 11));                     \
            p_[7] = __builtin_amdgcn_s_getreg(4 | (31 << 11));                      \
        }                                                                           \
    } while (0)

#else

#define ALNP_TL_VARS
#define ALNP_TL_MARK(k)
#define ALNP_TL_MARK_AFTER(k, value)
#define ALNP_TL_RECORD(row, waves)

#endif
