// Shared helpers of the CSA2 HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

// ---------------------------------------------------------------- host errors
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();
// Status of the launches enqueued just before (maps hipGetLastError).
csa2_status launch_status(const char* what);

#define CSA2_REQUIRE(cond, code, ...)   \
    do {                                \
        if (!(cond)) {                  \
            ::csa2::set_error(__VA_ARGS__); \
            return (code);              \
        }                               \
    } while (0)
#define CSA2_ARG(cond, ...) CSA2_REQUIRE(cond, CSA2_EINVAL, __VA_ARGS__)

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
inline int ilog2(int64_t v) {
    int s = 0;
    while ((int64_t(1) << s) < v) ++s;
    return s;
}

// ------------------------------------------------------------ row addressing
// Logical entry (b, j) -> physical row of a cache plane (contiguous slab per
// sequence, or pages of 2^page_shift entries through a page table).
struct RowMap {
    const int32_t* page_table;  // NULL -> contiguous
    int64_t seq_stride;
    int64_t capacity;           // entries addressable per sequence
    int32_t max_pages;
    int32_t page_shift;
};

__device__ __forceinline__ int64_t phys_row(const RowMap& m, int b, int64_t j) {
    if (m.page_table == nullptr) return (int64_t)b * m.seq_stride + j;
    int64_t page = m.page_table[(int64_t)b * m.max_pages + (j >> m.page_shift)];
    return (page << m.page_shift) + (j & ((int64_t(1) << m.page_shift) - 1));
}

// Validates a view's page geometry; fills the RowMap.
csa2_status make_rowmap(const int32_t* page_table, int32_t page_size, int32_t max_pages, int64_t seq_stride,
                        int64_t n_needed, RowMap* out, const char* what);

// ------------------------------------------------------------- device numerics
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

}  // namespace csa2
