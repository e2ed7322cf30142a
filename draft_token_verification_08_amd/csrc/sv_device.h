// sv_device.h -- device helpers shared by the kernels of libspecverify: DPP
// lane exchanges, the (value, lowest index) argmax and its 64-bit atomic key.
#pragma once

#include <hip/hip_runtime.h>

namespace sv {

__device__ __forceinline__ unsigned long long max64(unsigned long long* p, unsigned long long v) {
    return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lanes within a row of 16 exchange values with DPP (quad_perm, half-row and
// row mirrors); rows exchange with cross-lane shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

struct ArgMax {
    float v;
    int i;
};
__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
    // larger value wins; equal values keep the lower index
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

// 64-bit key whose unsigned order is the argmax order: order-preserving map of
// the float in the high word, the inverted index in the low word (equal values:
// the lower index has the larger key).  Zero is below every key of a number.
// -0.0 is keyed as +0.0: the two compare equal in better() and in the row
// scan's strict '>', so across chunks too the lower index must win between them.
__device__ __forceinline__ unsigned long long argmax_key(ArgMax a) {
    unsigned u = (a.v == 0.f) ? 0u : __float_as_uint(a.v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)u << 32) | (0xFFFFFFFFu - (unsigned)a.i);
}
__device__ __forceinline__ ArgMax argmax_unkey(unsigned long long k) {
    unsigned u = (unsigned)(k >> 32);
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return ArgMax{__uint_as_float(u), (int)(0xFFFFFFFFu - (unsigned)k)};
}

template <int CTRL>
__device__ __forceinline__ ArgMax dpp_am(ArgMax a) {
    return ArgMax{dpp_f<CTRL>(a.v), dpp_i<CTRL>(a.i)};
}

// argmax over each half wave (lanes 0-31 and 32-63); every lane of a half ends
// with its half's result
__device__ __forceinline__ ArgMax half_wave_argmax(ArgMax a) {
    a = better(a, dpp_am<kDppXor1>(a));
    a = better(a, dpp_am<kDppXor2>(a));
    a = better(a, dpp_am<kDppHalfMirror>(a));
    a = better(a, dpp_am<kDppMirror>(a));
    a = better(a, ArgMax{__shfl_xor(a.v, 16, 64), __shfl_xor(a.i, 16, 64)});
    return a;
}

}  // namespace sv
