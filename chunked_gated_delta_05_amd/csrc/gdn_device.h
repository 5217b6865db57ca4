// Device-side helpers shared by the HIP kernels of libgdn (forward and
// backward): vector types, the decay exponential, the LDS-only barrier, the
// unit map lookups and raw buffer resources. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// bits of a float. Taken through a by-value parameter: applied directly to a
// vector element (v[i]), __builtin_bit_cast reads element 0 with this
// compiler.
__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// b^x with the hardware base-2 exponential (about 1 ulp; e^x = 2^(x log2 e))
__device__ __forceinline__ float fpow(float x, int use_exp2) {
    return __builtin_amdgcn_exp2f(use_exp2 ? x : x * 1.4426950408889634f);
}

// The input transforms: beta through a sigmoid, and the reciprocal L2 norm
// of a q / k row from its sum of squares (epsilon 1e-6 under the root).
__device__ __forceinline__ float sigmoid_f(float x) {
    return 1.0f / (1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}
__device__ __forceinline__ float rnorm_f(float sumsq) { return 1.0f / __builtin_sqrtf(sumsq + 1e-6f); }

// Workgroup barrier for LDS hand-offs only: this wave's LDS accesses complete
// before it, but outstanding global loads and stores stay in flight (the
// fence of __syncthreads would wait for all of them).
// The s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8) waits for LDS only; it is issued through the
// builtin so that the compiler's own wait insertion knows what has completed.
constexpr int waitcnt_lgkm0() { return 15 | (3 << 14) | (7 << 4); }
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
    __builtin_amdgcn_s_barrier();
}

// ------------------------------------------------------------------ units
struct UnitInfo {
    int64_t start;   // first token on the flat axis
    int32_t len;     // tokens
    int32_t nch;     // chunks
    int32_t cbase;   // index of the unit's first chunk
};

__device__ __forceinline__ UnitInfo unit_info(const UnitMap& um, int u) {
    UnitInfo r;
    if (um.dense) {
        r.start = um.t_base + (int64_t)u * um.row_stride;
        r.len = um.T;
        r.nch = um.nt_dense;
        r.cbase = u * um.nt_dense;
        return r;
    }
    int64_t a = um.offsets[u], b = um.offsets[u + 1];
    a = a < 0 ? 0 : (a > um.total_tokens ? um.total_tokens : a);
    b = b < a ? a : (b > um.total_tokens ? um.total_tokens : b);
    r.start = a;
    r.len = (int32_t)(b - a);
    r.nch = (r.len + BT - 1) / BT;
    int cb = um.chunk_offsets[u];
    if (cb < 0) cb = 0;
    if (cb > um.n_chunks) cb = um.n_chunks;
    if (cb + r.nch > um.n_chunks) r.nch = um.n_chunks - cb;
    r.cbase = cb;
    return r;
}

// the same fields, marked wave-uniform (they depend on the workgroup only) so
// that values derived from them can live in scalar registers
__device__ __forceinline__ UnitInfo uniform(UnitInfo r) {
    const uint64_t s = (uint64_t)r.start;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)s), hi = __builtin_amdgcn_readfirstlane((uint32_t)(s >> 32));
    r.start = (int64_t)(((uint64_t)hi << 32) | lo);
    r.len = __builtin_amdgcn_readfirstlane(r.len);
    r.nch = __builtin_amdgcn_readfirstlane(r.nch);
    r.cbase = __builtin_amdgcn_readfirstlane(r.cbase);
    return r;
}

// (unit, chunk in unit) of a flat chunk index
__device__ __forceinline__ void chunk_of(const UnitMap& um, int ci, int& u, int& c) {
    if (um.dense) {
        u = ci / um.nt_dense;
        c = ci - u * um.nt_dense;
    } else {
        u = um.chunk_indices[2 * ci];
        c = um.chunk_indices[2 * ci + 1];
        if (u < 0 || u >= um.n_units) { u = -1; c = 0; }
    }
}

// raw buffer resource over [base, base + bytes): accesses outside read as zero
// and writes outside are dropped
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache policy of the output stores: non-temporal. A forward never reads o
// back, and o written through the caches would push k, q, v, T and P (which
// the next forward reads again) out of the last-level cache.
constexpr int CP_NT = 2;

}  // namespace gdn
