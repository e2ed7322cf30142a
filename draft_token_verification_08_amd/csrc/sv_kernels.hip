// sv_kernels.hip -- gfx950 kernels of libspecverify.
//
// The verify-and-sample step of "Accelerating Sonar through speculation"
// (Speculative decoding section: acceptance and target-generation stages;
// Target-draft section: acceptance compares the full draft and target
// distributions) with the acceptance test u < p/q and the residual max(0, p - q)
// of "Fast Inference from Transformers via Speculative Decoding", plus the MTP
// token shift/insert of the MTP and Single-token MTP scheduling sections.
//
// Passes (all on the caller's stream, no host synchronisation):
//   k_stats  one workgroup per (sequence, row slot, vocab chunk).  Streams its
//            chunk once with 16-byte loads and reduces it: greedy rows to
//            (max, lowest index), sampling rows to an online softmax partial
//            (chunk max m_c, sum of 2^((z - m_c) log2(e)/T)).  The last
//            workgroup of a sequence to finish (arrival counter) merges the
//            partials, runs the acceptance tests in order, finds the first
//            rejection and writes the accepted length and emitted tokens.
//            Target row L of a sampling sequence keeps per-tile partials for a
//            bonus draw.
//   k_draw   sampling sequences only.  Bonus draws (all drafts accepted): one
//            workgroup picks the tile of row L holding u*Z from the tile
//            partials and scans that tile.  Residual draws: one workgroup per
//            (sequence, draw chunk) sums max(0, p_k - q_k) per tile of its
//            chunk; the last workgroup of the sequence picks the tile holding
//            u*Z and scans only that tile.
//   k_mtp    token shift + insert and the hidden-state carry (16-byte copies).
//   The fused verify + MTP calls run no k_mtp: the decision shifts the token
//   buffer, the drawn token is written to both outputs, and every k_stats
//   workgroup copies an equal share of the hidden states after its rows.
//
// Determinism: every reduction has a fixed order (DPP/shuffle trees, then
// waves in order, then chunks in order); no floating-point atomics.
#include <cfloat>
#include <climits>
#include <cmath>

#include "sv_internal.h"
#include "sv_device.h"

#ifndef SV_ARGMAX_UNROLL
#define SV_ARGMAX_UNROLL 4
#endif
#ifndef SV_MS_UNROLL
#define SV_MS_UNROLL 4
#endif
#ifndef SV_NT_LOAD
#define SV_NT_LOAD 1
#endif
#ifndef SV_NT_COPY
#define SV_NT_COPY 0
#endif
#ifndef SV_COPY_VECS
#define SV_COPY_VECS 8  // 16-byte vectors per thread in the hidden-state copy
#endif
#ifndef SV_DRAW_WPE
#define SV_DRAW_WPE 5   // waves per SIMD the draw pass's registers are sized for
#endif
#ifndef SV_NEAR_Z
#define SV_NEAR_Z 0.01  // residual mass below which a draw takes the near form
#endif

namespace sv {

constexpr double kNearZ = SV_NEAR_Z;

// --------------------------------------------------------------- element access

// one 16-byte load of streamed logits (read once: optionally non-temporal)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const uint4* p) {
#if SV_NT_LOAD
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *p;
#endif
}

template <int DT> struct Elem;
template <> struct Elem<kBF16> { using T = uint16_t; static constexpr int kVec = 8; };
template <> struct Elem<kF32> { using T = float; static constexpr int kVec = 4; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT>
__device__ __forceinline__ float load_elem(const void* row, long long i) {
    if constexpr (DT == kBF16) {
        return __uint_as_float(((uint32_t)((const uint16_t*)row)[i]) << 16);
    } else {
        return ((const float*)row)[i];
    }
}

// Widen one 16-byte vector to floats (bf16 -> binary32 is exact: the 16 bits are
// the high half of the binary32 pattern).
template <int DT>
__device__ __forceinline__ void unpack(const uint4& w, float* f) {
    if constexpr (DT == kBF16) {
        f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
        f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
        f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
        f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
    } else {
        f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
        f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
    }
}

// a 16-byte vector of -inf (absent elements)
template <int DT>
__device__ __forceinline__ uint4 neg_inf_vec() {
    if constexpr (DT == kBF16) return make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
    else return make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u);
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const void* base, long long row, int V) {
    return (const char*)base + (size_t)row * (size_t)V * sizeof(typename Elem<DT>::T);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Row (in the target buffer) of target slot `slot` of sequence b: the slots of a
// sequence are R consecutive rows; with a row index, slot 0 is row row_index[b]
// clamped to [0, R) (only used with n = 0).
__device__ __forceinline__ long long target_row_of(int R, const int32_t* row_index, int b, int slot) {
    if (row_index == nullptr) return (long long)b * R + slot;
    int r = row_index[b];
    r = r < 0 ? 0 : (r >= R ? R - 1 : r);
    return (long long)b * R + r;
}

// --------------------------------------------------------------- cross-workgroup exchange
// Workgroups of one sequence hand their partial results to the last one to
// finish through device-scope atomic read-modify-writes only: the writer's data
// atomic returns before its arrival on the counter is performed, and the last
// workgroup reads (and resets to zero) the data with atomic exchanges.  No
// L2 writeback/invalidate fences are needed on the streaming workgroups.

__device__ __forceinline__ unsigned long long xchg64(unsigned long long* p, unsigned long long v) {
    return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned xchg32(unsigned* p, unsigned v) {
    return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Arrive on a counter after the data atomic whose returned value is `dep` has
// completed; returns the counter value before this arrival.
__device__ __forceinline__ unsigned arrive(unsigned* cnt, unsigned long long dep) {
    asm volatile("" ::"v"((unsigned)dep), "v"((unsigned)(dep >> 32)));
    __builtin_amdgcn_s_waitcnt(0);
    return __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long pack2(float a, float b) {
    return ((unsigned long long)__float_as_uint(b) << 32) | __float_as_uint(a);
}
__device__ __forceinline__ float lo_f(unsigned long long v) { return __uint_as_float((unsigned)v); }
__device__ __forceinline__ float hi_f(unsigned long long v) { return __uint_as_float((unsigned)(v >> 32)); }

// --------------------------------------------------------------- wave / block reductions
// Lanes within a row of 16 combine with DPP (quad_perm, half-row and row
// mirrors); rows combine with cross-lane shuffles (xor 16, xor 32).

__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
    a = better(a, dpp_am<kDppXor1>(a));
    a = better(a, dpp_am<kDppXor2>(a));
    a = better(a, dpp_am<kDppHalfMirror>(a));
    a = better(a, dpp_am<kDppMirror>(a));
    a = better(a, ArgMax{__shfl_xor(a.v, 16, 64), __shfl_xor(a.i, 16, 64)});
    a = better(a, ArgMax{__shfl_xor(a.v, 32, 64), __shfl_xor(a.i, 32, 64)});
    return a;
}

// online-softmax partial: (max, sum of 2^((z - max) * c))
struct MS {
    float m;
    float s;
};
__device__ __forceinline__ MS ms_combine(MS a, MS b, float c) {
    float m = fmaxf(a.m, b.m);
    float s = a.s * exp2_fast((a.m - m) * c) + b.s * exp2_fast((b.m - m) * c);
    return MS{m, s};
}
template <int CTRL>
__device__ __forceinline__ MS dpp_ms(MS a) {
    return MS{dpp_f<CTRL>(a.m), dpp_f<CTRL>(a.s)};
}
__device__ __forceinline__ MS wave_ms(MS a, float c) {
    a = ms_combine(a, dpp_ms<kDppXor1>(a), c);
    a = ms_combine(a, dpp_ms<kDppXor2>(a), c);
    a = ms_combine(a, dpp_ms<kDppHalfMirror>(a), c);
    a = ms_combine(a, dpp_ms<kDppMirror>(a), c);
    a = ms_combine(a, MS{__shfl_xor(a.m, 16, 64), __shfl_xor(a.s, 16, 64)}, c);
    a = ms_combine(a, MS{__shfl_xor(a.m, 32, 64), __shfl_xor(a.s, 32, 64)}, c);
    return a;
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
    v = max(v, dpp_i<kDppXor1>(v));
    v = max(v, dpp_i<kDppXor2>(v));
    v = max(v, dpp_i<kDppHalfMirror>(v));
    v = max(v, dpp_i<kDppMirror>(v));
    v = max(v, __shfl_xor(v, 16, 64));
    v = max(v, __shfl_xor(v, 32, 64));
    return v;
}

// Block reductions: waves in order 0..3 combined by thread 0; the result is
// valid in thread 0 only unless broadcast.
__device__ ArgMax block_argmax(ArgMax a) {
    __shared__ ArgMax sh[kWaves];
    a = wave_argmax(a);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh[w] = a;
    __syncthreads();
    ArgMax r = sh[0];
    if (threadIdx.x == 0)
        for (int i = 1; i < kWaves; ++i) r = better(r, sh[i]);
    return r;
}
__device__ MS block_ms(MS a, float c) {
    __shared__ MS sh[kWaves];
    a = wave_ms(a, c);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh[w] = a;
    __syncthreads();
    MS r = sh[0];
    if (threadIdx.x == 0)
        for (int i = 1; i < kWaves; ++i) r = ms_combine(r, sh[i], c);
    return r;
}
// Sum broadcast to every thread.
__device__ float block_sum_all(float v) {
    __shared__ float sh[kWaves];
    __shared__ float total;
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh[w] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = sh[0];
        for (int i = 1; i < kWaves; ++i) t += sh[i];
        total = t;
    }
    __syncthreads();
    return total;
}
__device__ int block_max_all(int v) {
    __shared__ int sh[kWaves];
    __shared__ int total;
    v = wave_max_i(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh[w] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = sh[0];
        for (int i = 1; i < kWaves; ++i) t = max(t, sh[i]);
        total = t;
    }
    __syncthreads();
    return total;
}

// --------------------------------------------------------------- per-thread row work

// Greedy: (max, lowest index) over elements [lo, hi) of one row.  Aligned path:
// thread t reads vectors t, t+256, ... in ascending order and keeps the first
// vector whose maximum beats its running maximum (index and contents, in
// registers: the streamed lines are not cached, so nothing is re-read); the lane
// inside that vector is resolved once at the end.
// The first group of thread_argmax's aligned loop (U vectors per thread), issued
// on its own so that a caller can start it before it knows the row is needed.
// Loads nothing when the range holds no full group.
template <int DT>
__device__ __forceinline__ void argmax_first_group(const void* row, int lo, int hi, uint4 (&w)[SV_ARGMAX_UNROLL]) {
    constexpr int kVec = Elem<DT>::kVec;
    constexpr int U = SV_ARGMAX_UNROLL;
    const int v = lo / kVec + (int)threadIdx.x, v1 = hi / kVec;
    if (v + (U - 1) * kThreads < v1) {
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = ld16((const uint4*)row + v + u * kThreads);
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// PRE: `pre` holds the first group, loaded by argmax_first_group on the same range.
template <int DT, bool ALIGNED, bool PRE = false>
__device__ ArgMax thread_argmax(const void* row, int lo, int hi, const uint4* pre = nullptr) {
    constexpr int kVec = Elem<DT>::kVec;
    const int tid = threadIdx.x;
    if constexpr (ALIGNED) {
        const uint4* vrow = (const uint4*)row;
        const int v0 = lo / kVec, v1 = hi / kVec;
        constexpr int U = SV_ARGMAX_UNROLL;
        float best = -INFINITY;
        int bestv = -1;
        uint4 bestw = make_uint4(0, 0, 0, 0);
        int v = v0 + tid;
        auto consume = [&](const uint4 (&w)[U], int vb) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[kVec];
                unpack<DT>(w[u], f);
                float m = f[0];
#pragma unroll
                for (int e = 1; e < kVec; ++e) m = fmaxf(m, f[e]);
                if (m > best) {
                    best = m;
                    bestv = vb + u * kThreads;
                    bestw = w[u];
                }
            }
        };
        if constexpr (PRE) {
            if (v + (U - 1) * kThreads < v1) {
                uint4 w[U];
#pragma unroll
                for (int u = 0; u < U; ++u) w[u] = pre[u];
                consume(w, v);
                v += U * kThreads;
            }
        }
        for (; v + (U - 1) * kThreads < v1; v += U * kThreads) {
            uint4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = ld16(vrow + v + u * kThreads);
            consume(w, v);
        }
        for (; v < v1; v += kThreads) {
            const uint4 w = ld16(vrow + v);
            float f[kVec];
            unpack<DT>(w, f);
            float m = f[0];
#pragma unroll
            for (int e = 1; e < kVec; ++e) m = fmaxf(m, f[e]);
            if (m > best) {
                best = m;
                bestv = v;
                bestw = w;
            }
        }
        ArgMax r{best, INT_MAX};
        if (bestv >= 0) {
            float f[kVec];
            unpack<DT>(bestw, f);
            int j = kVec - 1;
#pragma unroll
            for (int e = kVec - 1; e >= 0; --e)
                if (f[e] == best) j = e;
            r.i = bestv * kVec + j;
        } else if (v0 + tid < v1) {
            r.i = (v0 + tid) * kVec;  // every element -inf: the lowest own index
        }
        return r;
    } else {
        ArgMax r{-INFINITY, INT_MAX};
        for (int i = lo + tid; i < hi; i += kThreads) {
            const float x = load_elem<DT>(row, i);
            if (x > r.v || r.i == INT_MAX) r = ArgMax{x, i};  // first element, then strict '>'
        }
        return r;
    }
}

// Sampling: online softmax partial over [lo, hi) at c = log2(e)/T.  Per group of
// U vectors: take the group maximum, rescale the accumulators if it grew, then
// add 2^((z - m) c) with (z - m) formed first (exact for bf16 inputs).
template <int DT, bool ALIGNED>
__device__ MS thread_ms(const void* row, int lo, int hi, float c) {
    constexpr int kVec = Elem<DT>::kVec;
    const int tid = threadIdx.x;
    float m = -FLT_MAX;
    float acc[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[e] = 0.f;
    if constexpr (ALIGNED) {
        const uint4* vrow = (const uint4*)row;
        const int v0 = lo / kVec, v1 = hi / kVec;
        constexpr int U = SV_MS_UNROLL;
        int v = v0 + tid;
        for (; v + (U - 1) * kThreads < v1; v += U * kThreads) {
            uint4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = ld16(vrow + v + u * kThreads);
            float f[U][kVec];
#pragma unroll
            for (int u = 0; u < U; ++u) unpack<DT>(w[u], f[u]);
            float gm = m;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < kVec; ++e) gm = fmaxf(gm, f[u][e]);
            if (gm > m) {
                const float sc = exp2_fast((m - gm) * c);
#pragma unroll
                for (int e = 0; e < kVec; ++e) acc[e] *= sc;
                m = gm;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < kVec; ++e) acc[e] += exp2_fast((f[u][e] - m) * c);
        }
        for (; v < v1; v += kThreads) {
            float f[kVec];
            unpack<DT>(ld16(vrow + v), f);
            float gm = m;
#pragma unroll
            for (int e = 0; e < kVec; ++e) gm = fmaxf(gm, f[e]);
            if (gm > m) {
                const float sc = exp2_fast((m - gm) * c);
#pragma unroll
                for (int e = 0; e < kVec; ++e) acc[e] *= sc;
                m = gm;
            }
#pragma unroll
            for (int e = 0; e < kVec; ++e) acc[e] += exp2_fast((f[e] - m) * c);
        }
    } else {
        for (int i = lo + tid; i < hi; i += kThreads) {
            float x = load_elem<DT>(row, i);
            if (x > m) {
                acc[0] *= exp2_fast((m - x) * c);
                m = x;
            }
            acc[0] += exp2_fast((x - m) * c);
        }
    }
    float s = acc[0];
#pragma unroll
    for (int e = 1; e < kVec; ++e) s += acc[e];
    return MS{m, s};
}

// Elements [e0, e0 + kVec) of a row as floats; indices at or past `hi` read as
// -inf (never loaded).  e0 is a multiple of kVec.
template <int DT, bool ALIGNED>
__device__ __forceinline__ void load_vec(const void* row, int e0, int hi, float* f) {
    constexpr int kVec = Elem<DT>::kVec;
    if constexpr (ALIGNED) {
        if (e0 < hi) {
            unpack<DT>(ld16((const uint4*)row + e0 / kVec), f);
        } else {
#pragma unroll
            for (int e = 0; e < kVec; ++e) f[e] = -INFINITY;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) f[e] = (e0 + e < hi) ? load_elem<DT>(row, e0 + e) : -INFINITY;
    }
}

// The 16-byte vector of elements [e0, e0 + kVec) of a row whose base may not be
// 16-byte aligned, as raw bits (element by element); indices at or past `hi`
// hold -inf (never loaded).
template <int DT>
__device__ __forceinline__ uint4 load_raw(const void* row, int e0, int hi) {
    constexpr int kVec = Elem<DT>::kVec;
    unsigned w[4];
    if constexpr (DT == kBF16) {
        const uint16_t* r = (const uint16_t*)row;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned lo16 = (e0 + 2 * q < hi) ? r[e0 + 2 * q] : 0xff80u;
            const unsigned hi16 = (e0 + 2 * q + 1 < hi) ? r[e0 + 2 * q + 1] : 0xff80u;
            w[q] = lo16 | (hi16 << 16);
        }
    } else {
        const unsigned* r = (const unsigned*)row;
#pragma unroll
        for (int q = 0; q < kVec; ++q) w[q] = (e0 + q < hi) ? r[e0 + q] : 0xff800000u;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Sampling rows: softmax statistics over [lo, hi) (lo a multiple of the tile)
// in tiles of kThreads * kVec contiguous elements.  Wave w takes tiles w,
// w + kWaves, ...; inside a tile lane l reads vectors l, l + 64, l + 128, ...
// (coalesced).  Per tile: the wave maximum m_t, then s_t = sum 2^((z - m_t) c),
// each term formed as 2^fma(z, c, -fl(m_t c)) and the rounding of fl(m_t c)
// corrected once per tile (its exact residual is fma(m_t, c, -fl(m_t c))).
// Tile partials (m_t, s_t) are stored into `tiles` (when not null) for the
// bonus draw: with plain stores when the draw pass reads them (the kernel
// boundary orders them), with atomic exchanges, completed before the function
// returns, when `coherent` (the last workgroup of the sequence reads them in the
// same kernel).  The workgroup's merged (m, s) is returned in thread 0.
template <int DT, bool ALIGNED>
__device__ MS wg_softmax_tiles(const void* row, int lo, int hi, float c, unsigned long long* tiles,
                               bool coherent = false) {
    constexpr int kVec = Elem<DT>::kVec;
    constexpr int kTile = kThreads * kVec;
    constexpr int U = kThreads / 64;  // vectors per lane per tile
    __shared__ MS s_wave[kWaves];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t0 = lo / kTile, t1 = (hi + kTile - 1) / kTile;
    float M = -FLT_MAX, S = 0.f;
    unsigned long long dep = 0ull;
    // aligned rows: the next tile's 16-byte loads are issued before the current
    // tile is reduced (double buffer in registers); vectors past `hi` read -inf
    uint4 nxt[U];
    auto issue = [&](int tt) {
        if constexpr (ALIGNED) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = tt * kTile + (lane + 64 * u) * kVec;
                nxt[u] = (e0 < hi) ? ld16((const uint4*)row + e0 / kVec) : neg_inf_vec<DT>();
            }
        }
    };
    if (t0 + w < t1) issue(t0 + w);
    for (int t = t0 + w; t < t1; t += kWaves) {
        float f[U][kVec];
        if constexpr (ALIGNED) {
            uint4 cur[U];
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
            if (t + kWaves < t1) issue(t + kWaves);
#pragma unroll
            for (int u = 0; u < U; ++u) unpack<DT>(cur[u], f[u]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) load_vec<DT, ALIGNED>(row, t * kTile + (lane + 64 * u) * kVec, hi, f[u]);
        }
        float lm = f[0][0];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < kVec; ++e) lm = fmaxf(lm, f[u][e]);
        const float tmax = wave_max_f(lm);
        float ts = 0.f;
        if (tmax != -INFINITY) {
            const float mc = tmax * c;
            const float delta = fmaf(tmax, c, -mc);
            float acc[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) acc[e] = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < kVec; ++e) acc[e] += exp2_fast(fmaf(f[u][e], c, -mc));
            float ls = acc[0];
#pragma unroll
            for (int e = 1; e < kVec; ++e) ls += acc[e];
            ts = wave_sum(ls) * exp2_fast(-delta);
        }
        if (tiles != nullptr && lane == 0) {
            if (coherent) dep ^= xchg64(tiles + t, pack2(tmax, ts));
            else tiles[t] = pack2(tmax, ts);
        }
        const MS r = ms_combine(MS{M, S}, MS{tmax, ts}, c);
        M = r.m;
        S = r.s;
    }
    if (lane == 0) {
        if (coherent) {
            // this wave's tile exchanges have been performed before the barrier
            asm volatile("" ::"v"((unsigned)dep), "v"((unsigned)(dep >> 32)));
            __builtin_amdgcn_s_waitcnt(0);
        }
        s_wave[w] = MS{M, S};
    }
    __syncthreads();
    MS r = s_wave[0];
    if (threadIdx.x == 0)
        for (int i = 1; i < kWaves; ++i) r = ms_combine(r, s_wave[i], c);
    return r;
}

// --------------------------------------------------------------- inverse CDF
// Inverse CDF with unnormalised weights: y = the first index whose running sum
// exceeds t = u * Z.  Work is organised in tiles of kThreads * kVec contiguous
// elements (thread i of a tile owns elements [i*kVec, (i+1)*kVec) of it), tiles
// in chunks of kDrawTiles.  Every "which item holds t" question (chunk, tile,
// thread) is one block-wide prefix scan in binary64 (shuffle scan inside each
// wave, wave totals through LDS), run in passes of kThreads items.

struct Pick {
    int i;          // first item whose prefix range [before, before + w) holds t; -1 if none
    double before;  // prefix mass before item i
};

// Items 0..N-1, weight(i) >= 0 evaluated by thread i % kThreads in pass i / kThreads.
template <class W>
__device__ __forceinline__ Pick block_first_crossing(int N, double t, W&& weight) {
    __shared__ double s_wave[kWaves];
    __shared__ double s_pass_total;
    __shared__ int s_hit;
    __shared__ double s_before;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    double carry = 0.0;
    if (tid == 0) s_hit = INT_MAX;
    for (int base = 0; base < N; base += kThreads) {
        const int i = base + tid;
        const double wi = (i < N) ? weight(i) : 0.0;
        double incl = wi;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        if (lane == 63) s_wave[w] = incl;
        __syncthreads();
        double prev = carry;
        for (int k = 0; k < w; ++k) prev += s_wave[k];
        incl += prev;
        const double excl = incl - wi;
        if (wi > 0.0 && excl <= t && t < incl) atomicMin(&s_hit, i);
        if (tid == kThreads - 1) s_pass_total = incl;
        __syncthreads();
        const int hit = s_hit;
        if (hit != INT_MAX) {
            if (i == hit) s_before = excl;
            __syncthreads();
            return Pick{hit, s_before};
        }
        carry = s_pass_total;
        __syncthreads();
    }
    return Pick{-1, carry};
}

// 2^x - 1 for |x| <= 1/4: the exponential series in x ln 2 to degree 6, in
// Horner form (truncation below 3e-9 relative, binary32 rounding about 1e-7;
// exp2(x) - 1 would lose every digit as x -> 0).
__device__ __forceinline__ float exp2m1_small(float x) {
    float a = 1.5403530393381606e-04f;
    a = fmaf(a, x, 1.3333558146428441e-03f);
    a = fmaf(a, x, 9.618129107628477e-03f);
    a = fmaf(a, x, 5.5504108664821576e-02f);
    a = fmaf(a, x, 2.402265069591007e-01f);
    a = fmaf(a, x, 6.931471805599453e-01f);
    return a * x;
}

// Residual terms of one token in the near form, each row relative to its own
// maximum (at = z_t - m_t, ad = z_d - m_d, both <= 0 and exact for bf16 logits):
// A = 2^(at c), B = 2^(ad c) and the difference Dl = B - A in units of
// 2^(sl c), sl <= 0 a shift common to the row pair.  With x = (ad - at) c, Dl is
// formed as 2^((at - sl) c) (2^x - 1) when |x| <= 1/4 (no cancellation), else
// as 2^((ad - sl) c) - 2^((at - sl) c); a token whose relative logits agree
// (at = ad, masked in both rows included) has Dl = 0 exactly and no power of
// the shift is formed for it (only tokens with at != ad lie at or below sl).
// With S_t = sum A, S_d = sum B, rho = (S_d - S_t) 2^(-sl c) / S_t = sum Dl / S_t
// and lam = 1 + mu (B = A + 2^(sl c) Dl):
//   p - lam q = A / S_t - lam B / S_d = 2^(sl c) (kappa A - lam Dl) / S_d,
// kappa = rho - mu 2^(-sl c) (formed in binary64), so max(0, kappa A - lam Dl)
// are residual weights up to one common factor; the tokens the rows share never
// enter a difference, and their weight kappa A carries one rounding.
struct NearTerm {
    float A, Dl;
    float Bs;  // 2^((ad - sl) c), B in the units of Dl (0 for a token the rows share)
};
__device__ __forceinline__ float near_rel(float z, float m) { return m > -FLT_MAX ? z - m : -INFINITY; }
__device__ __forceinline__ NearTerm near_term(float m_t, float m_d, float sl, float c, float zt, float zd) {
    const float at = near_rel(zt, m_t), ad = near_rel(zd, m_d);
    const float A = exp2_fast(at * c);
    if (at == ad) return NearTerm{A, 0.f, 0.f};
    const float x = (ad - at) * c;
    const float As = exp2_fast((at - sl) * c);
    if (fabsf(x) <= 0.25f) {
        const float Dl = As * exp2m1_small(x);
        return NearTerm{A, Dl, As + Dl};
    }
    const float Bs = exp2_fast((ad - sl) * c);
    return NearTerm{A, Bs - As, Bs};
}
// The residual weight of one token in the near form (see near_term()).
__device__ __forceinline__ float near_weight(float m_t, float m_d, float sl, float c, float kappa, float lam, float zt,
                                            float zd) {
    const NearTerm t = near_term(m_t, m_d, sl, c, zt, zd);
    return fmaxf(fmaf(kappa, t.A, -lam * t.Dl), 0.f);
}

// How a draw weighs one element (all weights up to a factor common to the row):
//   kWTarget:   2^((z_t - mA) c), the target's own distribution (bonus draws, and
//               the fallback when no residual mass is left);
//   kWResFar:   max(0, P - lam Q) with P = 2^(z_t c - fl(m_t c)), Q = 2^(z_d c -
//               fl(m_d c)) (one rounding each: far_p()), each row scaled by its own
//               maximum (mA = m_t) and lam the ratio of their sums (S_t / S_d);
//   kWResNear:  near_weight(): max(0, kappa A - lam Dl) of near_term(), each
//               row relative to its own maximum (mA = m_t), differences in
//               units of 2^(sl c): the residual max(0, p - lam q);
//   kWResNearLog: the same weights formed from their log2 in binary64
//               (near_log_weight()) and scaled by 2^-E, for residuals whose
//               weights lie below the binary32 range in units of 2^(sl c);
//   kWTargetP:  the target's own distribution in the far form's units
//               P = 2^(z_t c - fl(m_t c)) (far_p()), for draws whose tile sums
//               were taken in those units.  The two target weightings differ by
//               the factor 2^(m_t c - fl(m_t c)), 1 + 1e-7 at ordinary
//               temperatures but up to 2 once m_t c passes 2^24 (T near 1e-6):
//               a draw scans its tile in the units its tile sums were taken in.
enum WMode : int { kWTarget = 0, kWResFar = 1, kWResNear = 2, kWResNearLog = 3, kWTargetP = 4 };
struct WSpec {
    int mode;
    float c;    // log2(e) / T
    float mA;   // maximum the target row is scaled by
    float m_d;  // kWResFar: the draft row's maximum
    float lam;    // kWResFar: lam S_t / S_d; kWResNear(Log): lam
    float kappa;  // kWResNear
    float sl;     // kWResNear(Log): the shift of the differences (<= 0)
    float nmt;  // kWResFar, kWTargetP: neg_scaled(mA, c)
    float nmd;  // kWResFar: neg_scaled(m_d, c)
    int ks;      // kWResNearLog: the sign of kappa (0: kappa = 0)
    double lk;   // kWResNearLog: log2 |kappa| (kappa in units of 2^(sl c))
    double sig;  // kWResNearLog: sl c
    double E;    // kWResNearLog: the weights' scale (an integer): weights are 2^(log2 w - E)
};
// -fl(m c) for a row maximum m, the offset of far_p(); 0 when the row has no
// finite element (m = -FLT_MAX), whose terms are then all 2^-inf = 0.
__device__ __forceinline__ float neg_scaled(float m, float c) { return m > -FLT_MAX ? -(m * c) : 0.f; }
// 2^(z c - fl(m c)) with nm = neg_scaled(m, c), one rounding (fma) before the
// power.  Every far-form sum and weight of a row pair takes its terms from here,
// so the rounding of fl(m c), a factor common to the whole row, cancels in the
// ratio lam = sum P / sum Q and in the normalised weights.
__device__ __forceinline__ float far_p(float nm, float c, float z) { return exp2_fast(fmaf(z, c, nm)); }
// log2(2^a + 2^b)
__device__ __forceinline__ double log2_add(double a, double b) {
    if (a == -INFINITY) return b;
    if (b == -INFINITY) return a;
    const double hi = fmax(a, b), lo = fmin(a, b);
    return hi + log2(1.0 + exp2(lo - hi));
}
// log2(1 - 2^y) for y <= 0 (-inf at 0), and log2(1 + 2^y): 1 - 2^y from the
// series of exp2m1_small() where |y| <= 1/4 (no digit lost), the logarithm by
// the hardware's log2.
__device__ __forceinline__ float log2_1m_exp2(float y) {
    const float v = y > -0.25f ? -exp2m1_small(y) : 1.f - exp2_fast(y);
    return __builtin_amdgcn_logf(v);
}
__device__ __forceinline__ float log2_1p_exp2(float y) { return __builtin_amdgcn_logf(1.f + exp2_fast(y)); }

// log2 of the near form's weight max(0, kappa A - lam Dl) of near_term() in
// units of 2^(sl c) (-inf: no weight).  The exponents (log2 A = at c, log2 |kappa|,
// the shift) are added in binary64, so that no weight leaves the range; the
// corrections of order 1 are binary32: lam |Dl| = lam 2^(at c - sl c) |2^x - 1|
// with x = (ad - at) c and |2^x - 1| = 2^max(x, 0) (1 - 2^-|x|), and sums and
// differences of two weights as 2^hi (1 +- 2^(lo - hi)).
__device__ __forceinline__ double near_log_weight(const WSpec& s, float zt, float zd) {
    const float at = near_rel(zt, s.mA), ad = near_rel(zd, s.m_d);
    if (at == -INFINITY) return -INFINITY;  // p = 0: max(0, -lam q) = 0
    const double ac = (double)at * (double)s.c;
    const double lkA = s.ks != 0 ? s.lk + ac : -INFINITY;  // log2 (|kappa| A)
    if (at == ad) return s.ks > 0 ? lkA : -INFINITY;
    const double x = ad == -INFINITY ? -INFINITY : ((double)ad - (double)at) * (double)s.c;
    const double lD = (double)__builtin_amdgcn_logf(s.lam) + ac - s.sig + fmax(x, 0.0) +
                      (double)log2_1m_exp2(-(float)fabs(x));
    if (x < 0.0) {  // target above draft: -lam Dl > 0
        if (s.ks > 0) {
            const double hi = fmax(lkA, lD), lo = fmin(lkA, lD);
            return hi + (double)log2_1p_exp2((float)(lo - hi));
        }
        if (s.ks < 0) return lkA < lD ? lD + (double)log2_1m_exp2((float)(lkA - lD)) : -INFINITY;
        return lD;
    }
    return (s.ks > 0 && lkA > lD) ? lkA + (double)log2_1m_exp2((float)(lD - lkA)) : -INFINITY;
}

// An upper bound of near_log_weight() from the exponents alone, in binary32
// with a margin e = 1 + 2^-20 (|at c| + |sl c| + |log2 |kappa||) for the
// roundings of its handful of operations: within 1 + 2e of the weight where the
// target's logit exceeds the draft's.  lkf = log2 |kappa|, sgf = sl c, llf =
// log2 lam.  Where the draft's exceeds the target's by x = (ad - at) c >= 1, the
// weight is positive only if log2 |kappa| + sl c - log2 lam > x + log2(1 - 2^-x)
// >= x - 1.
__device__ __forceinline__ float near_log_bound(int ks, float lkf, float sgf, float llf, float c, float m_t,
                                                float m_d, float zt, float zd) {
    const float at = near_rel(zt, m_t), ad = near_rel(zd, m_d);
    if (at == -INFINITY) return -INFINITY;
    const float ac = at * c;
    const float e = 1.f + 0x1p-20f * (fabsf(ac) + fabsf(sgf) + fabsf(lkf));
    const float lkA = ks != 0 ? lkf + ac : -INFINITY;
    if (ad < at) return fmaxf(lkA, llf + ac - sgf) + 1.f + e;
    if (ks <= 0) return -INFINITY;
    if (ad == at) return lkA + e;
    const float x = (ad - at) * c;
    return (x >= 1.f + e && x - 1.f - e >= lkf + sgf - llf) ? -INFINITY : lkA + e;
}

__device__ __forceinline__ float elem_weight(const WSpec& s, float zt, float zd) {
    if (s.mode == kWTarget) return exp2_fast((zt - s.mA) * s.c);
    if (s.mode == kWTargetP) return far_p(s.nmt, s.c, zt);
    if (s.mode == kWResNearLog) {
        const double lw = near_log_weight(s, zt, zd);
        return lw == -INFINITY ? 0.f : exp2_fast((float)(lw - s.E));
    }
    if (s.mode == kWResFar) {
        const float P = far_p(s.nmt, s.c, zt);
        const float Q = far_p(s.nmd, s.c, zd);
        return fmaxf(fmaf(-s.lam, Q, P), 0.f);
    }
    return near_weight(s.mA, s.m_d, s.sl, s.c, s.kappa, s.lam, zt, zd);
}
__device__ __forceinline__ WSpec target_spec(const DrawDesc& d) {
    return WSpec{kWTarget, d.c, d.m_t, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
}
__device__ __forceinline__ WSpec target_p_spec(const DrawDesc& d) {
    return WSpec{kWTargetP, d.c, d.m_t, 0.f, 0.f, 0.f, 0.f, neg_scaled(d.m_t, d.c), 0.f};
}
__device__ __forceinline__ bool target_only(const WSpec& s) { return s.mode == kWTarget || s.mode == kWTargetP; }

// Scan one tile: returns the element whose running weight (starting at P)
// first exceeds t.  The thread holding t is picked from per-thread sums taken in
// binary64 over the same terms the element scan adds, so the two agree; if
// rounding still leaves t unreached inside that thread, its last element of
// positive weight is taken (the neighbour of the boundary).  If t lies past the
// whole tile (or take_last), the tile's last element of positive weight is
// taken, or the tile's first element when it has none.
template <int DT, bool ALIGNED>
__device__ __forceinline__ int scan_tile(const WSpec& ws, const void* trow, const void* drow, int V, int tile,
                                         double P, double t, bool take_last) {
    constexpr int kVec = Elem<DT>::kVec;
    constexpr int kTile = kThreads * kVec;
    const int e0 = tile * kTile + threadIdx.x * kVec;
    const bool residual = !target_only(ws);
    float zt[kVec], zd[kVec], wv[kVec];
    load_vec<DT, ALIGNED>(trow, e0, V, zt);
    if (residual) load_vec<DT, ALIGNED>(drow, e0, V, zd);
    double ts = 0.0;
    int my_last = -1;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        wv[e] = (e0 + e < V) ? elem_weight(ws, zt[e], residual ? zd[e] : 0.f) : 0.f;
        ts += (double)wv[e];
        if (wv[e] > 0.f) my_last = e0 + e;
    }
    __shared__ double s_ts[kThreads];
    __shared__ int s_y;
    s_ts[threadIdx.x] = ts;
    if (threadIdx.x == 0) s_y = -1;
    __syncthreads();
    Pick pk{-1, 0.0};
    if (!take_last) pk = block_first_crossing(kThreads, t - P, [&](int i) { return s_ts[i]; });
    if (pk.i == (int)threadIdx.x) {
        double run = P + pk.before;
        int y = my_last;  // t unreached through rounding: the boundary's neighbour
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            run += (double)wv[e];
            if (run > t && wv[e] > 0.f) {
                y = e0 + e;
                break;
            }
        }
        s_y = y;
    }
    const int last = block_max_all(my_last);
    __syncthreads();
    int y = s_y;
    if (y < 0) y = (last >= 0) ? last : tile * kTile;
    return y;
}

// --------------------------------------------------------------- MTP helpers

__device__ __forceinline__ u32x4 ld_copy(const u32x4* p) {
#if SV_NT_COPY
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
__device__ __forceinline__ void st_copy(u32x4* p, u32x4 v) {
#if SV_NT_COPY
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// Copy vectors [v0, v1) of src to dst with the workgroup: coalesced, four
// 16-byte loads in flight per thread.
__device__ __forceinline__ void copy_range(const u32x4* src, u32x4* dst, long long v0, long long v1) {
    long long v = v0 + threadIdx.x;
#pragma unroll 1
    for (; v + 3 * kThreads < v1; v += 4 * kThreads) {
        const u32x4 w0 = ld_copy(src + v), w1 = ld_copy(src + v + kThreads);
        const u32x4 w2 = ld_copy(src + v + 2 * kThreads), w3 = ld_copy(src + v + 3 * kThreads);
        st_copy(dst + v, w0);
        st_copy(dst + v + kThreads, w1);
        st_copy(dst + v + 2 * kThreads, w2);
        st_copy(dst + v + 3 * kThreads, w3);
    }
    for (; v < v1; v += kThreads) st_copy(dst + v, ld_copy(src + v));
}

// Workgroup `part` of `nparts` copies its share of the hidden states: whole
// units of kThreads vectors, split as evenly as the unit count allows.
__device__ __forceinline__ void copy_share(const MtpFuse& m, long long part, long long nparts) {
    if (m.hsrc == nullptr || m.nvec <= 0) return;
    const long long units = (m.nvec + kThreads - 1) / kThreads;
    const long long q = units / nparts, r = units % nparts;
    const long long u0 = q * part + (part < r ? part : r);
    const long long u1 = u0 + q + (part < r ? 1 : 0);
    const long long v0 = u0 * kThreads;
    const long long v1 = u1 * kThreads < m.nvec ? u1 * kThreads : m.nvec;
    if (v0 < v1) copy_range((const u32x4*)m.hsrc, (u32x4*)m.hdst, v0, v1);
}

// Token shift of sequence b (slot i <- slot i + 1 for i < n; slot n kept).
__device__ __forceinline__ void shift_tokens(int32_t* tokens, int b, int n) {
    int32_t* t = tokens + (size_t)b * (n + 1);
    for (int i = 0; i < n; ++i) t[i] = t[i + 1];
}

// Draw from the target row's own distribution (the bonus token from p_L after
// full acceptance): pick the tile holding u * Z from the tile partials (m_t, s_t)
// the stats pass stored for this row, weighted on the scale 2^((z - m) c) of the
// row maximum m, with one block prefix scan; then scan only that tile.
// ATOMIC: the partials are read, and reset to zero, with atomic exchanges (the
// stats pass's own decision); else with plain loads (the draw pass, which
// clears them afterwards).
template <int DT, bool ALIGNED, bool ATOMIC>
__device__ __forceinline__ int tile_draw(unsigned long long* tiles, int NT, int V, const DrawDesc& d,
                                         const void* trow, double* s_w /* LDS, >= kMaxTiles */) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    double mine = 0.0;
    int my_last = -1;
    for (int i = tid; i < NT; i += kThreads) {
        const unsigned long long q = ATOMIC ? xchg64(tiles + i, 0ull) : tiles[i];
        const float ts = hi_f(q);
        const double wi = ts > 0.f ? (double)ts * exp2(((double)lo_f(q) - (double)d.m_t) * (double)d.c) : 0.0;
        s_w[i] = wi;
        mine += wi;
        if (wi > 0.0) my_last = i;
    }
    __shared__ double s_part[kWaves];
    __shared__ double s_t;
    __shared__ int s_last_tile;
    double incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_part[w] = incl;
    const int last_tile = block_max_all(my_last);
    if (tid == 0) {
        double Z = 0.0;
        for (int k = 0; k < kWaves; ++k) Z += s_part[k];
        s_t = (double)d.u * Z;
        s_last_tile = last_tile < 0 ? 0 : last_tile;
    }
    __syncthreads();
    const double t = s_t;
    const Pick pk = block_first_crossing(NT, t, [&](int i) { return s_w[i]; });
    const WSpec ws = target_spec(d);
    if (pk.i >= 0) return scan_tile<DT, ALIGNED>(ws, trow, nullptr, V, pk.i, pk.before, t, false);
    return scan_tile<DT, ALIGNED>(ws, trow, nullptr, V, s_last_tile, 0.0, t, true);
}

// --------------------------------------------------------------- decision helpers

__device__ __forceinline__ int clamp_len(int L, int n, uint32_t& flags) {
    if (L < 0) { flags |= SV_FLAG_LEN_CLAMPED; L = 0; }
    if (L > n) { flags |= SV_FLAG_LEN_CLAMPED; L = n; }
    return L;
}

__device__ __forceinline__ double sanitize_u(float uf, uint32_t& flags) {
    double u = (double)uf;
    if (!(u >= 0.0)) { flags |= SV_FLAG_BAD_UNIFORM; return 0.0; }
    if (u >= 1.0) { flags |= SV_FLAG_BAD_UNIFORM; return 1.0 - 5.9604644775390625e-08; }
    return u;
}

// log2(e) / T, kept finite so that (z - m) * c stays well defined for tiny T.
__device__ __forceinline__ float exp2_scale(float T) {
    float c = 1.4426950408889634f / T;
    return fminf(c, FLT_MAX);
}

// Per-sequence settings every workgroup of a sequence derives identically.
struct SeqInfo {
    int L;          // effective draft length
    float T;        // temperature (sanitised)
    bool greedy;    // greedy rule for this sequence
    uint32_t flags; // flags raised while deriving the above
};

template <int MODE>
__device__ __forceinline__ SeqInfo seq_info(const StatsParams& p, int b) {
    SeqInfo s;
    s.flags = 0;
    s.L = (p.lens != nullptr) ? clamp_len(p.lens[b], p.n, s.flags) : 0;
    if (p.row_index != nullptr && (p.row_index[b] < 0 || p.row_index[b] >= p.R)) s.flags |= SV_FLAG_ROW_CLAMPED;
    s.T = 0.f;
    s.greedy = true;
    if constexpr (MODE == kSample) {
        float T = p.temp[b];
        if (!(T >= 0.f)) { s.flags |= SV_FLAG_BAD_TEMP; T = 0.f; }
        s.T = T;
        s.greedy = !(T > 0.f);
        if (!s.greedy && p.draft == nullptr && s.L > 0) {
            // no draft logits: nothing can be verified, plain sampling of one token
            s.flags |= SV_FLAG_LEN_CLAMPED;
            s.L = 0;
        }
    }
    return s;
}

// Greedy tree verification of sequence b ("Accelerating Sonar through
// speculation", EAGLE section: the target scores the candidate sequences of the
// draft tree, the longest suitable one is kept and one more target token is
// appended).  Node 0 is the root; node j + 1 (j < L) holds draft token x_j
// below node parents[j] in [0, j] (other parents leave the node out, flagged).
// Node i is accepted iff its parent is and x_{i-1} is the target's argmax g at
// the parent (g[r] = argmax of target row r, lowest index on ties).  The kept
// path ends at the deepest accepted node, the lowest-numbered among equally deep
// ones; its tokens are emitted, then g of its last node, then -1.
//
// One wave does it, lane j holding node j + 1 (L <= 64), with no serial walk:
// pointer doubling (6 rounds of shuffles) gives every node its depth and whether
// every edge up to the root matches, a wave max picks the kept node, and binary
// lifting over the doubling's ancestor tables (6 more rounds) tells each node
// whether it lies on the kept path, so each writes its own output slot.
__device__ __forceinline__ void tree_walk(const StatsParams& p, int b, const SeqInfo& si, const int* s_idx) {
    constexpr int kLog = 6;  // 2^6 = kMaxDraft: the longest root path
    static_assert((1 << kLog) == kMaxDraft && kMaxDraft == 64, "one wave64 holds the tree");
    const int j = threadIdx.x, n = p.n, V = p.V, L = si.L;
    if (j >= 64) return;  // waves 1..3: nothing left to do
    const int i = j + 1;  // this lane's node
    const bool live = j < L;
    const int x = live ? p.tokens[(size_t)b * n + j] : 0;
    const int par = live ? p.parents[(size_t)b * n + j] : 0;
    const bool good = live && par >= 0 && par < i;
    const unsigned long long oor = __ballot(live && (x < 0 || x >= V));
    const unsigned long long bad = __ballot(live && !good);

    // (a, ok, d): an ancestor a of node i (0 once the root is reached), whether
    // every edge from i up to a matches, and how many edges that is.
    int a = good ? par : 0;
    const int gp = s_idx[good ? par : 0];  // g at the parent (row 0 when none)
    int ok = good && x == gp;
    int d = 1;
    int up[kLog];  // up[k]: the ancestor 2^k edges above node i (0 past the root)
#pragma unroll
    for (int k = 0; k < kLog; ++k) {
        up[k] = a;
        const int src = a > 0 ? a - 1 : j;
        const int a2 = __shfl(a, src, 64), ok2 = __shfl(ok, src, 64), d2 = __shfl(d, src, 64);
        if (a > 0) {
            ok &= ok2;
            d += d2;
            a = a2;
        }
    }
    // after 64 edges every path has met the root: ok = accepted, d = depth
    const int key = wave_max_i(good && ok ? (d << 7) | (127 - j) : 0);
    const int k = key >> 7;                          // depth of the kept node
    const int best = key ? 128 - (key & 127) : 0;   // its node index (0: the root)

    // binary lifting: the ancestor of `best` at this node's depth
    int node = best;
    const int lift = k - d;
#pragma unroll
    for (int t = 0; t < kLog; ++t) {
        const int src = node > 0 ? node - 1 : j;
        const int nu = __shfl(up[t], src, 64);
        if (node > 0 && lift >= 0 && ((lift >> t) & 1)) node = nu;
    }
    int32_t* e = p.emitted + (size_t)b * (n + 1);
    int32_t* path = p.path ? p.path + (size_t)b * n : nullptr;
    if (good && ok && lift >= 0 && node == i) {  // on the kept path, at depth d
        e[d - 1] = x;
        if (path) path[d - 1] = i;
    }
    for (int t = k + j; t <= n; t += 64) e[t] = t == k ? s_idx[best] : -1;
    if (path)
        for (int t = k + j; t < n; t += 64) path[t] = -1;
    if (j == 0) {
        p.acc[b] = k;
        const uint32_t flags = si.flags | (oor ? SV_FLAG_TOKEN_OOR : 0u) | (bad ? SV_FLAG_BAD_PARENT : 0u);
        if (flags && p.flags) atomicOr(p.flags, flags);
        xchg32(&p.cnt[b], 0u);  // leave the counter zero for the next call
    }
}

// --------------------------------------------------------------- sampling tree walks
// Sampling tree verification ("Accelerating Sonar through speculation", EAGLE
// section: the target scores the draft's candidate tree, the longest suitable
// sequence is kept, one target token appended), with SpecInfer's multi-step
// speculative sampling as the acceptance rule.  At node u the children are
// tested in index order against the current target residual: child j + 1 is
// accepted iff u[j] < max(0, p_u(x) - lam q_u(x)) / (M q_u(x)), where after k
// rejections at u lam = lam_k and M = M_k = sum max(0, p_u - lam_k q_u)
// (lam_0 = 0, M_0 = 1, lam_{k+1} = lam_k + M_k).  An accepted child moves the
// walk down; with no child left the token is drawn from max(0, p_u - lam q_u)
// (from p_u itself when u has no children).  The first test at a node needs
// only the rows' statistics; each later one needs the residual at lam_k, a full
// reduction of the pair (p_u, q_u), which a round kernel provides (the test's
// ratio and log2 M_k, RoundStep): the walk then stops, pending.  lam_k - 1 is
// kept as log2 (lmu), so that a residual mass below binary64's resolution at 1
// (T -> 0, rows on one top token) still enters lam, and with it a lower bound
// of the next residual's mass (zb), which picks the draw's form.  The weight of
// the tokens whose relative logits agree in both rows is kappa_k 2^(a c) / S_d
// with kappa_k = S_d / S_t - lam_k; after the second rejection it can be a
// product of two tails, far below the binary64 resolution of lam_k, so the walk
// carries kappa_k itself from the round that formed M_k (sign and log2).

// One sequence's walk inputs, staged in LDS: statistics of target rows (mt, St)
// and draft rows (md, Sd) by node, and node j + 1's token, parent (-1 when not
// an earlier node) and gathered logits gt = z_t[parent][x_j], gd = z_d[parent][x_j].
struct WalkRows {
    const float* mt;
    const double* St;
    const float* md;
    const double* Sd;
    const float* gt;
    const float* gd;
    const int* x;
    const int* par;
};

// The first acceptance ratio at node u, of node j + 1: p_u(x) / q_u(x) formed in
// log space as the linear decision forms it (so it keeps its value when both
// probabilities are below the binary64 range).
__device__ double tree_ratio(const WalkRows& r, int j, int u, int V, float c) {
    const int x = r.x[j];
    if (x < 0 || x >= V) return 0.0;
    const float zt = r.gt[j], zd = r.gd[j];
    if (zt == -INFINITY) return 0.0;
    if (zd == -INFINITY) return INFINITY;
    const double cd = (double)c;
    const double lr = ((double)zt - (double)r.mt[u]) * cd - ((double)zd - (double)r.md[u]) * cd;
    return exp2(lr) * (r.Sd[u] / r.St[u]);
}

// What one round hands the walk for the one test it makes possible: the
// pending child's acceptance ratio under the residual at the current lam_k,
// (p_u(x) - lam_k q_u(x)) / (M_k q_u(x)), log2 M_k for lam_{k+1} = lam_k + M_k,
// and kappa_{k+1} = S_d / S_t - lam_{k+1} as sign and log2 (next_kappa()).
struct RoundStep {
    double ratio, lM, lkap;
    int skap;
};

// DrawDesc::mu from log2(lam - 1), and back: log2 mu, and mu (0 below binary64)
__device__ __forceinline__ double encode_mu(double lmu) {
    if (lmu == -INFINITY) return 0.0;
    return lmu >= -1000.0 ? exp2(lmu) : lmu;
}
__device__ __forceinline__ double desc_lmu(const DrawDesc& d) {
    if (d.mu == 0.0) return -INFINITY;
    return d.mu > 0.0 ? log2(d.mu) : d.mu;
}
__device__ __forceinline__ double desc_mu(const DrawDesc& d) { return d.mu > 0.0 ? d.mu : 0.0; }

// A signed quantity s 2^l (s = +1 or -1, l = -inf: zero), for kappa = S_d / S_t
// - lam, which after later rejections at a tree node is a product of tails and
// may lie below the binary64 range.
struct SLog2 {
    int s;
    double l;
};
// a + b, the difference formed as 2^hi (1 - 2^(lo - hi)) with expm1 (no digit lost to 1 - 2^d)
__device__ __forceinline__ SLog2 slog2_add(SLog2 a, SLog2 b) {
    if (a.l == -INFINITY) return b;
    if (b.l == -INFINITY) return a;
    const SLog2 hi = a.l >= b.l ? a : b, lo = a.l >= b.l ? b : a;
    const double dd = lo.l - hi.l;
    if (hi.s == lo.s) return SLog2{hi.s, hi.l + log2(1.0 + exp2(dd))};
    if (dd == 0.0) return SLog2{1, -INFINITY};
    return SLog2{hi.s, hi.l + log2(-expm1(dd * 0.6931471805599453))};
}
__device__ __forceinline__ SLog2 slog2_of(double v) { return SLog2{v < 0.0 ? -1 : 1, v != 0.0 ? log2(fabs(v)) : -INFINITY}; }
// kappa carried by a tree walk (d.skap != 0), in units of 2^lu (0 below binary64)
__device__ __forceinline__ double desc_kappa(const DrawDesc& d, double lu) {
    return d.lkap == -INFINITY ? 0.0 : (double)d.skap * exp2(d.lkap - lu);
}

// A lower bound of the residual mass sum max(0, p - q) after a rejection of x:
// q(x) - p(x), and from the rows' sums (S = sum 2^((z - m) c), so each row's top
// token has probability 1 / S) |1 / S_t - 1 / S_d| (the target's top token gives
// p - q >= 1 / S_t - 1 / S_d, the draft's q - p >= 1 / S_d - 1 / S_t, and the
// mass is both sum max(0, p - q) and sum max(0, q - p)).  A draw whose bound is
// below the near form's threshold hands over the near form's sums
// (kDrawResidualNear).  After a later rejection at a tree node (lam_{k+1} =
// lam_k + M_k) the mass is M_k times that of max(0, r_k - q) with r_k the
// residual the child was tested against, so M_k (q(x) - r_k(x)) bounds it, and
// so does M_k (q(y) - r_k(y)) at the draft's top token y, where q(y) = 1 / S_d and
// M_k r_k(y) = max(0, p(y) - lam_k / S_d) <= max(0, 1 / S_t - lam_k / S_d); the
// target's top token gives 1 / S_t - lam_{k+1} / S_d.
__device__ __forceinline__ double resid_mass_bound(double St, double Sd, double gap) {
    return fmax(gap, fabs(1.0 / St - 1.0 / Sd));
}

// Runs the walk from its state (one thread).  Returns true when it has
// finished: *d then describes the draw (kDrawTarget at a node with no child
// left and no rejection, else a residual draw at the walk's lam).  Returns false,
// with the state pending, when the next test needs the residual at the current
// lam and no round's result for that test (`step`, when have_step) is left (only if
// can_pend; otherwise the children not yet tested are left out, which is the
// same rule on a smaller tree, and SV_FLAG_TREE_TRUNCATED is raised).
__device__ __forceinline__ bool tree_walk_run(TreeWalk& w, const WalkRows& r, int L, int V, const float* uni,
                                              bool can_pend, RoundStep step, bool have_step, DrawDesc* d) {
    for (;;) {
        int j = -1;
        for (int t = w.next; t < L; ++t)
            if (r.par[t] == w.u) {
                j = t;
                break;
            }
        if (j < 0) {  // no child left to test at u
            const int u = w.u;
            *d = DrawDesc{};
            d->k = u;
            d->slot = w.depth;
            d->c = w.c;
            d->m_t = r.mt[u];
            if (w.zb < 0.0) {
                d->kind = kDrawTarget;
                d->m_d = r.mt[u];
            } else {
                d->kind = w.zb < kNearZ ? kDrawResidualNear : kDrawResidual;
                d->m_d = r.md[u];
                d->lq = (float)log2(r.St[u] / r.Sd[u]);
                d->mu = encode_mu(w.lmu);
                d->skap = w.skap;
                d->lkap = w.lkap;
            }
            w.status = kWalkIdle;
            return true;
        }
        double ratio, lM = -INFINITY;
        SLog2 kn{0, -INFINITY};  // kappa after this child's rejection (a round's result)
        if (w.zb < 0.0) {
            ratio = tree_ratio(r, j, w.u, V, w.c);
        } else if (have_step) {  // the round's result is for this child
            ratio = step.ratio;
            lM = step.lM;
            kn = SLog2{step.skap, step.lkap};
            have_step = false;
        } else {  // the residual at lam not formed yet
            if (can_pend) {
                w.next = j;
                w.status = kWalkPending;
                return false;
            }
            w.flags |= SV_FLAG_TREE_TRUNCATED;
            w.next = L;
            continue;
        }
        const double uj = sanitize_u(uni[j], w.flags);
        if (uj < ratio) {  // accepted: one level down
            w.path[w.depth++] = j + 1;
            w.u = j + 1;
            w.zb = -1.0;
            w.lmu = -INFINITY;
            w.skap = 0;
            w.lkap = -INFINITY;
        } else {
            // q_u(x) (1 - the ratio x was tested at): the rejected child's share of
            // the next residual mass (resid_mass_bound())
            const int x = r.x[j];
            double gap = 0.0;
            if (x >= 0 && x < V && r.gd[j] > -INFINITY)
                gap = exp2(((double)r.gd[j] - (double)r.md[w.u]) * (double)w.c) / r.Sd[w.u] * (1.0 - fmin(ratio, 1.0));
            if (w.zb < 0.0) {  // first rejection: lam_1 = lam_0 + M_0 = 1
                w.zb = resid_mass_bound(r.St[w.u], r.Sd[w.u], gap);
                w.lmu = -INFINITY;
            } else {  // the residual loses q_u once more: lam_{k+1} = lam_k + M_k
                // 1 / S_t - lam / S_d = kappa / S_d, from the carried kappa once there is one
                const double St = r.St[w.u], Sd = r.Sd[w.u], Mk = exp2(lM);
                const double k_now = w.skap != 0 ? (w.lkap == -INFINITY ? 0.0 : w.skap * exp2(w.lkap))
                                                 : Sd / St - 1.0;
                const double k_next = kn.l == -INFINITY ? 0.0 : kn.s * exp2(kn.l);
                w.zb = fmax(Mk * gap, fmax(Mk / Sd - fmax(0.0, k_now / Sd), k_next / Sd));
                w.lmu = log2_add(w.lmu, lM);
                w.skap = kn.s != 0 ? kn.s : 1;
                w.lkap = kn.l;
            }
        }
        w.next = j + 1;
    }
}

// Writes a finished walk's outputs (accepted length, emitted prefix, -1 in the
// drawn slot and after it, the path) and its draw descriptor; one thread.
__device__ void tree_walk_finish(const TreeWalk& w, DrawDesc d, const int* x, int n, float u_final, int32_t* acc,
                                 int32_t* emitted, int32_t* path, DrawDesc* desc, uint32_t* flags, int b) {
    uint32_t f = w.flags;
    d.u = (float)sanitize_u(u_final, f);
    desc[b] = d;
    acc[b] = w.depth;
    int32_t* e = emitted + (size_t)b * (n + 1);
    for (int i = 0; i <= n; ++i) e[i] = i < w.depth ? x[w.path[i] - 1] : -1;
    if (path)
        for (int i = 0; i < n; ++i) path[(size_t)b * n + i] = i < w.depth ? w.path[i] : -1;
    if (f && flags) atomicOr(flags, f);
}

// Stores (pending) or clears (finished) a walk's persistent state: the walk and
// its rows block, which stay zero while no walk is pending.
__device__ void tree_walk_store(const TreeWalk& w, bool pending, const WalkRows& r, int L, int n, TreeWalk* gw,
                                char* rows) {
    const TreeRowsLayout lay = tree_rows_layout(n);
    float* mt = reinterpret_cast<float*>(rows + lay.mt);
    double* St = reinterpret_cast<double*>(rows + lay.St);
    float* md = reinterpret_cast<float*>(rows + lay.md);
    double* Sd = reinterpret_cast<double*>(rows + lay.Sd);
    float* gt = reinterpret_cast<float*>(rows + lay.gt);
    float* gd = reinterpret_cast<float*>(rows + lay.gd);
    for (int i = 0; i <= L; ++i) {
        mt[i] = pending ? r.mt[i] : 0.f;
        St[i] = pending ? r.St[i] : 0.0;
    }
    for (int i = 0; i < L; ++i) {
        md[i] = pending ? r.md[i] : 0.f;
        Sd[i] = pending ? r.Sd[i] : 0.0;
        gt[i] = pending ? r.gt[i] : 0.f;
        gd[i] = pending ? r.gd[i] : 0.f;
    }
    if (pending) *gw = w;
    else *gw = TreeWalk{};
}

// The statistics pass's decision for a sampling tree (T > 0): stage the walk's
// rows (statistics merged in LDS, gathered logits), flag bad parents and tokens,
// run the walk from the root.
__device__ void tree_sample_decide(const StatsParams& p, int b, const SeqInfo& si, float* s_m, double* s_S,
                                   const void* target, const void* draft, bool bf16) {
    __shared__ int s_x[kMaxDraft], s_par[kMaxDraft];
    __shared__ float s_gt[kMaxDraft], s_gd[kMaxDraft];
    const int tid = threadIdx.x, n = p.n, V = p.V, L = si.L;
    uint32_t bad = 0;
    if (tid < 64) {
        const int j = tid;
        bool oor = false, badp = false;
        if (j < L) {
            const int x = p.tokens[(size_t)b * n + j];
            const int par = p.parents[(size_t)b * n + j];
            badp = !(par >= 0 && par <= j);
            oor = x < 0 || x >= V;
            float gt = -INFINITY, gd = -INFINITY;
            if (!badp && !oor) {
                const size_t tr = (size_t)b * (n + 1) + par, dr = (size_t)b * n + par;
                if (bf16) {
                    gt = __uint_as_float(((uint32_t)((const uint16_t*)target)[tr * V + x]) << 16);
                    gd = __uint_as_float(((uint32_t)((const uint16_t*)draft)[dr * V + x]) << 16);
                } else {
                    gt = ((const float*)target)[tr * V + x];
                    gd = ((const float*)draft)[dr * V + x];
                }
            }
            s_x[j] = x;
            s_par[j] = badp ? -1 : par;
            s_gt[j] = gt;
            s_gd[j] = gd;
        }
        const unsigned long long mo = __ballot(oor), mb = __ballot(badp);
        bad = (mo ? (uint32_t)SV_FLAG_TOKEN_OOR : 0u) | (mb ? (uint32_t)SV_FLAG_BAD_PARENT : 0u);
    }
    __shared__ TreeWalk s_walk;  // the walk's state (LDS: its path is indexed at run time)
    __shared__ uint32_t s_bad;
    if (tid == 0) s_bad = bad;
    __syncthreads();
    if (tid == 0) {
        const WalkRows r{s_m, s_S, s_m + n + 1, s_S + n + 1, s_gt, s_gd, s_x, s_par};
        TreeWalk& w = s_walk;
        w = TreeWalk{};
        w.u = 0;
        w.zb = -1.0;
        w.lmu = -INFINITY;
        w.skap = 0;
        w.lkap = -INFINITY;
        w.c = exp2_scale(si.T);
        w.flags = si.flags | s_bad;
        DrawDesc d;
        const float* uni = p.unif + (size_t)b * (n + 1);
        if (tree_walk_run(w, r, L, V, uni, p.can_pend != 0, RoundStep{0.0, 0.0, -INFINITY, 0}, false, &d))
            tree_walk_finish(w, d, s_x, n, uni[n], p.acc, p.emitted, p.path, p.desc, p.flags, b);
        else
            tree_walk_store(w, true, r, L, n, p.walk + b, p.trows + (size_t)b * tree_rows_layout(n).stride);
        xchg32(&p.cnt[b], 0u);  // leave the counter zero for the next call
    }
}

// The greedy decision of sequence b after its argmax keys are merged (g[r] in
// s_idx): the longest prefix of drafts equal to g, then g at the first mismatch.
// One wave writes the outputs, lane j its own emitted slot and, with the fused
// MTP step, its own token slot (t[j] = t[j + 1] for j < n, then t[k] = g[k]);
// every lane's load of t[j + 1] completes before any lane's store, since the
// stores take their data from those loads.
__device__ __forceinline__ void greedy_finish(const StatsParams& p, int b, const SeqInfo& si, const int* s_idx) {
    const int j = threadIdx.x, n = p.n, V = p.V, L = si.L;
    if (j >= 64) return;  // waves 1..3: nothing left to do
    const int x = j < L ? p.tokens[(size_t)b * n + j] : 0;
    const bool oor = j < L && (x < 0 || x >= V);
    const bool rej = j < L && (oor || x != s_idx[j]);
    const unsigned long long rmask = __ballot(rej);
    const unsigned long long omask = __ballot(oor);
    const int k = rmask ? __ffsll((long long)rmask) - 1 : L;  // first rejection, or L
    const int g = s_idx[k];
    int32_t* e = p.emitted + (size_t)b * (n + 1);
    if (j <= n) e[j] = j < k ? x : (j == k ? g : -1);
    if (n == kMaxDraft && j == 0) e[n] = k == n ? g : -1;
    if (p.mtp.tokens) {
        int32_t* t = p.mtp.tokens + (size_t)b * (n + 1);
        const int next = j < n ? t[j + 1] : 0;
        if (j < n) t[j] = j == k ? g : next;
        if (k == n && j == 0) t[n] = g;
    }
    if (j == 0) {
        uint32_t f = si.flags;
        const unsigned long long upto = (k >= 63) ? ~0ull : ((2ull << k) - 1ull);  // slots 0..k
        if (omask & upto) f |= SV_FLAG_TOKEN_OOR;
        p.acc[b] = k;
        if (f && p.flags) atomicOr(p.flags, f);
        xchg32(&p.cnt[b], 0u);  // leave the counter zero for the next call
    }
}

// The decision of sequence b, run by the last workgroup of b to finish.  DRAW
// (calls with no drafts): it also makes the bonus draw.  TREE (greedy): the
// drafts form a tree, and the kept path is found by tree_walk.
template <int DT, int MODE, bool ALIGNED, bool DRAW = false, bool TREE = false>
__device__ void decide(const StatsParams& p, int b, const SeqInfo& si) {
    __shared__ float s_m[kMaxSlots];
    __shared__ double s_S[kMaxSlots];
    __shared__ int s_idx[kMaxSlots];

    const int tid = threadIdx.x;
    const int n = p.n, V = p.V, NC = p.NC, S = p.S, L = si.L;
    const float cf = si.greedy ? 0.f : exp2_scale(si.T);
    const double cd = (double)cf;
    unsigned long long* part = reinterpret_cast<unsigned long long*>(p.part) + (size_t)b * S * NC;
    __shared__ unsigned long long s_part[kMaxPartials];

    // 1. collect (and reset to zero) the partials of every row read, then merge
    //    them per row in ascending chunk order
    if (MODE == kGreedy || si.greedy) {
        // one argmax key per row (chunk slot 0), already merged by atomic max
        if (tid <= L) {
            const ArgMax r = argmax_unkey(xchg64(part + (size_t)tid * NC, 0ull));
            s_m[tid] = r.v;
            s_idx[tid] = r.i;
        }
    } else {
        for (int i = tid; i < S * NC; i += kThreads) s_part[i] = xchg64(part + i, 0ull);
        __syncthreads();
        const bool draft_row = tid > n && tid < S && tid - n - 1 < L;
        const bool row_read = (tid <= L) || (draft_row && p.dstats == nullptr);
        if (draft_row && p.dstats != nullptr) {
            // statistics the draft's sampling step computed over the same row at the same T
            const float* ds = p.dstats + ((size_t)b * n + (tid - n - 1)) * 2;
            s_m[tid] = ds[0];
            s_S[tid] = (double)ds[1];
        }
        if (row_read) {
            // online merge in double: running max, rescaled sum
            float m = -FLT_MAX;
            double Ssum = 0.0;
            for (int c = 0; c < NC; ++c) {
                const unsigned long long q = s_part[tid * NC + c];
                const float mc = lo_f(q), sc = hi_f(q);
                if (mc > m) {
                    Ssum *= exp2((double)(m - mc) * cd);
                    m = mc;
                }
                Ssum += (double)sc * exp2((double)(mc - m) * cd);
            }
            s_m[tid] = m;
            s_S[tid] = Ssum;
        }
    }
    __syncthreads();
    if constexpr (TREE) {
        if (MODE == kGreedy || si.greedy) tree_walk(p, b, si, s_idx);
        else tree_sample_decide(p, b, si, s_m, s_S, p.target, p.draft, DT == kBF16);
        return;
    }
    if constexpr (MODE == kGreedy) {
        greedy_finish(p, b, si, s_idx);
        return;
    }
    if constexpr (MODE == kSample) {
        if (p.row_lse && tid < 2 * n + 1) {
            const bool row_read = !si.greedy && ((tid <= L) || (tid > n && tid - n - 1 < L));
            float v = __builtin_nanf("");
            if (row_read) v = (float)((double)s_m[tid] / (double)si.T + log(s_S[tid]));
            p.row_lse[(size_t)b * (2 * n + 1) + tid] = v;
        }
        if (p.out_stats && tid == 0) {
            const float nan = __builtin_nanf("");
            p.out_stats[(size_t)b * 2] = si.greedy ? nan : s_m[0];
            p.out_stats[(size_t)b * 2 + 1] = si.greedy ? nan : (float)s_S[0];
        }
    }
    __syncthreads();

    // 2. the acceptance tests: lane j of wave 0 tests draft slot j (n <= 64); a
    //    wave ballot of the rejections and find-first-set give the first
    //    rejection k (slots past k are evaluated but unused)
    __shared__ int s_k;
    __shared__ uint32_t s_flags;
    __shared__ double s_gap;
    if (tid < 64) {
        const int j = tid;
        bool rej = false, oor = false, badu = false;
        double gap = 0.0;  // q(x) - p(x), a lower bound of the residual mass after rejecting x
        int x = 0;
        if constexpr (!DRAW) x = j < L ? p.tokens[(size_t)b * n + j] : 0;
        if (j < L) {
            if constexpr (DRAW) x = p.tokens[(size_t)b * n + j];
            if (x < 0 || x >= V) {
                oor = true;
                rej = true;
            } else if (si.greedy) {
                rej = (x != s_idx[j]);
            } else {
                const float zt = load_elem<DT>(row_ptr<DT>(p.target, target_row_of(p.R, p.row_index, b, j), V), x);
                const float zd = load_elem<DT>(row_ptr<DT>(p.draft, (long long)b * n + j, V), x);
                uint32_t fl = 0;
                const double u = sanitize_u(p.unif[(size_t)b * (n + 1) + j], fl);
                badu = (fl != 0);
                const int jd = n + 1 + j;
                double ratio;
                const bool pz = (zt == -INFINITY), qz = (zd == -INFINITY);
                if (qz) ratio = pz ? 0.0 : INFINITY;
                else if (pz) ratio = 0.0;
                else {
                    // p/q = 2^((zt - m_t) c) / S_t  /  (2^((zd - m_d) c) / S_d)
                    const double lr = ((double)zt - (double)s_m[j]) * cd - ((double)zd - (double)s_m[jd]) * cd;
                    ratio = exp2(lr) * (s_S[jd] / s_S[j]);
                }
                if (!qz) gap = exp2(((double)zd - (double)s_m[jd]) * cd) / s_S[jd] * (1.0 - fmin(ratio, 1.0));
                rej = !(u < ratio);
            }
        }
        const unsigned long long rmask = __ballot(rej);
        const unsigned long long omask = __ballot(oor);
        const unsigned long long bmask = __ballot(badu);
        const int k = rmask ? __ffsll((long long)rmask) - 1 : L;
        const unsigned long long upto = (k >= 63) ? ~0ull : ((2ull << k) - 1ull);  // slots 0..k
        if constexpr (!DRAW) {
            // the emitted prefix and the fused MTP token shift, lane j its own
            // slots (as in greedy_finish); slot k: g for greedy sequences, else
            // the draw pass's
            const int yk = si.greedy ? s_idx[k] : -1;
            int32_t* e = p.emitted + (size_t)b * (n + 1);
            if (j <= n) e[j] = j < k ? x : (j == k ? yk : -1);
            if (n == kMaxDraft && j == 0) e[n] = k == n ? yk : -1;
            if (p.mtp.tokens) {
                int32_t* t = p.mtp.tokens + (size_t)b * (n + 1);
                const int next = j < n ? t[j + 1] : 0;
                if (j < n) t[j] = (j == k && si.greedy) ? yk : next;
                if (k == n && si.greedy && j == 0) t[n] = yk;
            }
        }
        if (j == k) s_gap = gap;
        if (tid == 0) {
            uint32_t f = si.flags;
            if (omask & upto) f |= SV_FLAG_TOKEN_OOR;
            if (bmask & upto) f |= SV_FLAG_BAD_UNIFORM;
            s_k = k;
            s_flags = f;
        }
    }
    __syncthreads();

    // 3. emitted tokens; sampling sequences: the draw descriptor
    __shared__ DrawDesc s_desc;
    if (tid == 0) {
        uint32_t flags = s_flags;
        const int k = s_k;
        // calls with no drafts write their outputs here, from one thread (the
        // wave-wide writes above measured slower in that kernel's code)
        int32_t* e = p.emitted + (size_t)b * (n + 1);
        if constexpr (DRAW) {
            const int32_t* x = p.tokens + (size_t)b * n;
            for (int j = 0; j < k; ++j) e[j] = x[j];
            for (int j = k + 1; j <= n; ++j) e[j] = -1;
        }
        p.acc[b] = k;
        if constexpr (DRAW)
            if (p.mtp.tokens) shift_tokens(p.mtp.tokens, b, n);  // fused MTP step
        if (si.greedy) {
            if constexpr (DRAW) {
                e[k] = s_idx[k];
                if (p.mtp.tokens) p.mtp.tokens[(size_t)b * (n + 1) + k] = s_idx[k];
            }
        } else {
            const double u = sanitize_u(p.unif[(size_t)b * (n + 1) + n], flags);
            // the draw (residual after a rejection, bonus after full acceptance)
            // is done by the draw pass
            if constexpr (DRAW) e[k] = -1;
            DrawDesc d{};  // skap = 0: kappa = S_d / S_t - 1, formed by the draw
            // a rejection whose residual mass may lie below the near form's
            // threshold (resid_mass_bound()) hands the draw the near form's sums
            const double zb = (k < L) ? resid_mass_bound(s_S[k], s_S[n + 1 + k], s_gap) : 0.0;
            d.kind = (k < L) ? (zb < kNearZ ? kDrawResidualNear : kDrawResidual) : kDrawBonus;
            d.k = k;
            d.slot = k;
            d.c = cf;
            d.m_t = s_m[k];
            d.m_d = (k < L) ? s_m[n + 1 + k] : 0.f;
            d.lq = (k < L) ? (float)log2(s_S[k] / s_S[n + 1 + k]) : 0.f;
            d.u = (float)u;
            d.mu = 0.0;
            if constexpr (DRAW) s_desc = d;  // drawn below, by this workgroup
            else p.desc[b] = d;
        }
        if (flags && p.flags) atomicOr(p.flags, flags);
        xchg32(&p.cnt[b], 0u);  // leave the counter zero for the next call
    }
    if constexpr (MODE == kSample && DRAW) {
        // calls with no drafts (n = 0): every draw is a bonus draw from target
        // row 0, made here from its tile partials (exchanged atomically by the
        // row's workgroups) instead of by the draw pass, which is not launched
        if (!si.greedy) {
            __syncthreads();
            const DrawDesc d = s_desc;
            const void* trow = row_ptr<DT>(p.target, target_row_of(p.R, p.row_index, b, d.k), V);
            const int y = tile_draw<DT, ALIGNED, true>(p.tiles + (size_t)b * p.NT, p.NT, V, d, trow,
                                                       reinterpret_cast<double*>(s_part));
            if (tid == 0) {
                p.emitted[(size_t)b * (n + 1) + d.slot] = y;
                if (p.mtp.tokens) p.mtp.tokens[(size_t)b * (n + 1) + d.slot] = y;
            }
        }
    }
}

// --------------------------------------------------------------- stats pass

// The parameters are taken by value: taken by reference, the inlined sampling
// pass compiled to different code that measured 13% slower at B=256, n=4.
template <int DT, int MODE, bool ALIGNED, bool DRAW, bool TREE = false>
__device__ __forceinline__ void stats_pass(StatsParams p) {
    const int bid = blockIdx.x;
    const int c = bid % p.NC;
    const int rest = bid / p.NC;
    const int slot = rest % p.S;
    const int b = rest / p.S;
    const int n = p.n;
    const int lo = c * p.CH;
    const int hi = min(p.V, lo + p.CH);

    // Greedy launches read target rows only, and every slot <= n lies inside the
    // [B][n+1][V] target buffer: the first load group is issued before the draft
    // length says whether the row is needed (the values are used only if it is).
    uint4 pre[SV_ARGMAX_UNROLL];
    if constexpr (MODE == kGreedy && ALIGNED)
        argmax_first_group<DT>(row_ptr<DT>(p.target, target_row_of(p.R, p.row_index, b, slot), p.V), lo, hi, pre);

    const SeqInfo si = seq_info<MODE>(p, b);
    const bool target_row = slot <= n;
    const bool needed =
        target_row ? (slot <= si.L) : (!si.greedy && p.dstats == nullptr && slot - n - 1 < si.L);
    if (!needed) {
        copy_share(p.mtp, bid, gridDim.x);
        return;
    }
    const unsigned expected =
        (unsigned)p.NC * (unsigned)(si.L + 1 + ((si.greedy || p.dstats != nullptr) ? 0 : si.L));

    const void* row = target_row ? row_ptr<DT>(p.target, target_row_of(p.R, p.row_index, b, slot), p.V)
                                 : row_ptr<DT>(p.draft, (long long)b * n + (slot - n - 1), p.V);
    unsigned long long* slot_part =
        reinterpret_cast<unsigned long long*>(p.part) + ((size_t)b * p.S + slot) * p.NC;
    __shared__ int s_last;
    if (si.greedy) {
        ArgMax t;
        if constexpr (MODE == kGreedy && ALIGNED) t = thread_argmax<DT, ALIGNED, true>(row, lo, hi, pre);
        else t = thread_argmax<DT, ALIGNED>(row, lo, hi);
        const ArgMax r = block_argmax(t);
        if (threadIdx.x == 0) {
            const unsigned long long dep = max64(slot_part, argmax_key(r));  // merged across chunks
            s_last = (arrive(&p.cnt[b], dep) == expected - 1u);
        }
    } else {
        const float cf = exp2_scale(si.T);
        // sampling tree: the draft row of a node with no child is never used (no
        // test is made and no residual formed there), so it is not read
        bool skip = false;
        if constexpr (TREE) {
            if (!target_row) {
                const int k = slot - n - 1, j = threadIdx.x;
                skip = !__syncthreads_or(j < si.L && j >= k && p.parents[(size_t)b * n + j] == k);
            }
        }
        // target row L is the only row a bonus token can be drawn from: it alone
        // streams in tiles and keeps per-tile partials
        const MS r = skip ? MS{-INFINITY, 0.f}
                     : (target_row && slot == si.L && !TREE)
                         ? wg_softmax_tiles<DT, ALIGNED>(row, lo, hi, cf, p.tiles + (size_t)b * p.NT, DRAW)
                         : block_ms(thread_ms<DT, ALIGNED>(row, lo, hi, cf), cf);
        if (threadIdx.x == 0) {
            const unsigned long long dep = xchg64(slot_part + c, pack2(r.m, r.s));
            s_last = (arrive(&p.cnt[b], dep) == expected - 1u);
        }
    }
    __syncthreads();
    if (s_last) decide<DT, MODE, ALIGNED, DRAW, TREE>(p, b, si);
    // fused MTP step: every workgroup of the grid carries an equal share of the
    // hidden states once its row chunk is done (the copy's writes then come as
    // one burst at the end of the read stream instead of interleaved with it)
    copy_share(p.mtp, bid, gridDim.x);
}

// The statistics pass (one workgroup per (sequence, row slot, vocab chunk)).
template <int DT, int MODE, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k_stats(StatsParams p) {
    stats_pass<DT, MODE, ALIGNED, false>(p);
}
// Greedy tree verification: the greedy statistics pass over the tree's node
// rows, then the tree walk.
template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k_stats_tree(StatsParams p) {
    stats_pass<DT, kGreedy, ALIGNED, false, true>(p);
}
// Sampling tree verification: the sampling statistics pass over the tree's node
// rows, then the walk from the root.
template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k_stats_tree_sample(StatsParams p) {
    stats_pass<DT, kSample, ALIGNED, false, true>(p);
}
// Sampling calls with no drafts: the statistics pass whose decision also makes
// the (bonus) draw, so no draw pass follows.
template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k_stats_draw(StatsParams p) {
    stats_pass<DT, kSample, ALIGNED, true>(p);
}


// --------------------------------------------------------------- draw pass
// Bonus draws (all drafts accepted): workgroup (b, 0) alone, with tile_draw().
// Residual draws (draft k rejected) from max(0, p_k - q_k): workgroup (b, c)
// reads its chunk of kDrawTiles tiles of target row k and draft row k once
// (thread i: vector i of every tile) and hands over per-tile sums by atomic
// exchange; the last workgroup of the sequence picks the tile holding u * Z with
// one block prefix scan and scans only that tile.
//
// The weights are max(0, P - lam Q), each row scaled by its own maximum
// (kWResFar), with lam = S_t / S_d taken from the same P and Q terms: the chunks
// hand over, per tile, sum P, sum Q, and at the statistics pass's estimate lam0
// the weight sum W = sum max(0, P - lam0 Q) and its slope G = sum Q over the
// tokens with P > lam0 Q.  The last workgroup forms lam = sum P / sum Q and each
// tile's weight W - (lam - lam0) G (exact unless a token's P / Q lies between
// lam0 and lam).  Each weight then carries binary32 rounding relative to P and
// lam Q, not to their difference: measured, the normalised CDF error of these
// weights is about 3e-8 / Z for residual mass Z = sum W / sum P.  When Z is
// below kNearZ (the draft is almost the target, or T -> 0 with both rows on one
// top token) the weights take the near form, in which the tokens the rows share
// cancel exactly.  The decision marks the draws whose mass may be that small
// (resid_mass_bound()), and their chunks hand over the near form's sums instead
// (near_lin()).  Where those cannot settle the tile weights (the mass below what
// the statistics' sums resolve, or below the binary32 range), and for an
// unmarked draw whose far-form mass turns out small, the last workgroup re-forms
// the pair's weights by itself (near_exact_tiles(): the differences scaled to
// the largest of them, the pair read three times): slow, but reached with
// probability about Z_k <= 1e-6.
constexpr int kSumP = 0, kSumQ = 1, kSumW = 2, kSumG = 3;

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
// Two sums over the workgroup, the same value in every thread.
__device__ void block_sum2_all(double& a, double& b) {
    __shared__ double sh[2][kWaves];
    a = wave_sum_d(a);
    b = wave_sum_d(b);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        sh[0][w] = a;
        sh[1][w] = b;
    }
    __syncthreads();
    a = sh[0][0];
    b = sh[1][0];
    for (int i = 1; i < kWaves; ++i) {
        a += sh[0][i];
        b += sh[1][i];
    }
    __syncthreads();
}

// Per-element accumulation of a residual tile's far-form sums (lane-private, in
// the order the caller visits the elements); the draw pass and the parity/debug
// kernel both use it, so both form the same sums.
struct FarSums {
    float p, q, w, g;
};
__device__ __forceinline__ void far_accum(FarSums& s, float nmt, float nmd, float c, float lam0, float zt, float zd) {
    const float P = far_p(nmt, c, zt);
    const float Q = far_p(nmd, c, zd);
    const float w0 = fmaf(-lam0, Q, P);
    s.p += P;
    s.q += Q;
    s.w += fmaxf(w0, 0.f);
    s.g += w0 > 0.f ? Q : 0.f;
}
__device__ __forceinline__ FarSums wave_far_sums(FarSums s) {
    return FarSums{wave_sum(s.p), wave_sum(s.q), wave_sum(s.w), wave_sum(s.g)};
}
__device__ __forceinline__ float far_sum_at(const FarSums& s, int q) {
    return q == kSumP ? s.p : q == kSumQ ? s.q : q == kSumW ? s.w : s.g;
}

// The near form handed over by a draw's chunks (kDrawResidualNear): its weights
// max(0, kappa A - lam Dl) (near_term() with no shift) are linear in kappa
// between the tokens' crossing points, so the chunks hand over, per tile, sum A,
// sum Dl, and at the estimate kappa0 = rho0 - mu (rho0 = S_d / S_t - 1 from the
// statistics pass, one binary32 rounding of lq) the weight sum W and its slope
// G = sum A over the tokens with a positive weight; the deciding workgroup forms
// kappa = sum Dl / sum A - mu and each tile's weight W + (kappa - kappa0) G.
// That is exact unless a token's crossing point lies between kappa0 and kappa;
// the tokens the rows share all cross at kappa = 0, which the plan keeps apart.
// A tree walk's round needs kappa after the next rejection too, which the
// chunks' sums give without a difference of nearly equal numbers (next_kappa()):
// per tile they also hand over, over the tokens whose relative logits differ,
// sum B and the sum of the positive weights at kappa0.  After two or more
// rejections at a node the walk carries kappa itself (DrawDesc::skap), and
// kappa0 is that value.
constexpr int kSumA = 0, kSumDl = 1;   // near form: the slots of sum P and sum Q
constexpr int kSumY = 4, kSumWd = 5;   // near form only
struct NearSums {
    float a, dl, w, g, y, wd;
};
__device__ __forceinline__ NearSums wave_near_sums(NearSums s) {
    return NearSums{wave_sum(s.a), wave_sum(s.dl), wave_sum(s.w), wave_sum(s.g), wave_sum(s.y), wave_sum(s.wd)};
}
__device__ __forceinline__ float near_sum_at(const NearSums& s, int q) {
    return q == 0 ? s.a : q == 1 ? s.dl : q == 2 ? s.w : q == 3 ? s.g : q == 4 ? s.y : s.wd;
}
struct NearLin {
    float kappa0, lam;
};
__device__ __forceinline__ NearLin near_lin(const DrawDesc& d) {
    const double mu = desc_mu(d);
    if (d.skap != 0) return NearLin{(float)desc_kappa(d, 0.0), (float)(1.0 + mu)};
    const double rho0 = fabs((double)d.lq) <= 0.25 ? (double)exp2m1_small(-d.lq) : exp2(-(double)d.lq) - 1.0;
    return NearLin{(float)(rho0 - mu), (float)(1.0 + mu)};
}
__device__ __forceinline__ void near_accum(NearSums& s, const DrawDesc& d, const NearLin& nl, float zt, float zd) {
    // near_term() with no shift (the powers of (a - 0) c are those of a c)
    const float at = near_rel(zt, d.m_t), ad = near_rel(zd, d.m_d);
    const float A = exp2_fast(at * d.c);
    float Dl = 0.f, B = 0.f;
    if (at != ad) {
        const float x = (ad - at) * d.c;
        if (fabsf(x) <= 0.25f) {
            Dl = A * exp2m1_small(x);
            B = A + Dl;
        } else {
            B = exp2_fast(ad * d.c);
            Dl = B - A;
        }
    }
    const float w0 = fmaf(nl.kappa0, A, -nl.lam * Dl);
    s.a += A;
    s.dl += Dl;
    s.w += fmaxf(w0, 0.f);
    s.g += w0 > 0.f ? A : 0.f;
    s.y += B;
    s.wd += (at != ad && w0 > 0.f) ? w0 : 0.f;
}

// What plan_residual() decided besides the tile weights and the element
// weighting: Z the total of the tile weights (at or below zero: no residual
// mass left, -Z the target's own total), mass = sum max(0, p - lam q) in
// binary64 (0 where it lies below that range) and lmass its log2 (kept there;
// -inf: none), sq the draft row's sum in the weights' units (far form sum Q,
// near form S_d in A's units), and the near form's kappa and lam in binary64.
struct ResidPlan {
    double Z, mass, lmass, sq, kappa, lam;
    double sh;   // near form: 2^(-sl c), the unit of its differences (binary64; may be +inf)
    bool exact;  // the near form by the deciding workgroup alone (near_exact_tiles())
    // near form, for next_kappa(): over the tokens whose relative logits differ,
    // yd = sum B and lwd = log2 sum max(0, kappa A - lam Dl), in units of 2^lu
    // (lu = sl c, 0 for the chunks' sums); kappa in those units as sign ks and
    // log2 |kappa| lk
    double yd, lwd, lu, lk;
    int ks;
};

// The near form of one row pair, formed by one workgroup from the rows
// themselves (near_term()): first the shift sl = max(at, ad) over the tokens
// whose relative logits differ (-inf when none does: p = q), then
// S_t = sum A, rho = sum Dl / S_t and Y = sum B over the differing tokens, then
// each tile's weight sum max(0, kappa A - lam Dl) into s_w[NT], the residual
// max(0, p - lam q) at lam = 1 + mu (kappa carried by a tree walk, else
// rho - mu 2^(-sl c)), in binary32 or, where that range cannot hold them, from
// their log2 (near_log_weight()).  Fills *ws (element weighting) and *pl
// (ResidPlan, with the sums next_kappa() needs).  Wave w takes tiles w,
// w + kWaves, ...; lane l the vectors l, l + 64, ... of a tile.
__device__ float block_max_f_all(float v) {
    __shared__ float sh[kWaves];
    v = wave_max_f(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh[w] = v;
    __syncthreads();
    v = sh[0];
    for (int i = 1; i < kWaves; ++i) v = fmaxf(v, sh[i]);
    __syncthreads();
    return v;
}
// Two maxima over the workgroup, the same values in every thread.
__device__ void block_max2_d_all(double& a, double& b) {
    __shared__ double sh[2][kWaves];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a = fmax(a, __shfl_xor(a, off, 64));
        b = fmax(b, __shfl_xor(b, off, 64));
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        sh[0][w] = a;
        sh[1][w] = b;
    }
    __syncthreads();
    a = sh[0][0];
    b = sh[1][0];
    for (int i = 1; i < kWaves; ++i) {
        a = fmax(a, sh[0][i]);
        b = fmax(b, sh[1][i]);
    }
    __syncthreads();
}
template <int DT, bool ALIGNED>
__device__ void near_exact_tiles(const void* trow, const void* drow, int V, int NT, const DrawDesc& d, double* s_w,
                                 WSpec* ws, ResidPlan* pl, bool need_next) {
    constexpr int kVec = Elem<DT>::kVec;
    constexpr int kTile = kThreads * kVec;
    constexpr int kU = kThreads / 64;
    constexpr int kH = ALIGNED ? kU : 1;  // vectors per row in flight
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const float c = d.c, m_t = d.m_t, m_d = d.m_d;
    // calls f(zt, zd) for the elements of vectors u0 .. u0 + kH - 1 of tile t
    // (absent elements -inf).  The element math is long: unrolled over a
    // vector it would set the kernel's register count, so the elements are
    // visited one 32-bit word of each row at a time (aligned rows, all loads
    // issued before the first use) or one element at a time (element-wise loads).
    auto visit = [&](int t, int u0, auto&& f) {
        if constexpr (ALIGNED) {
            uint4 wt[kH], wd[kH];
#pragma unroll
            for (int h = 0; h < kH; ++h) {
                const int e0 = t * kTile + (lane + 64 * (u0 + h)) * kVec;
                wt[h] = e0 < V ? ld16((const uint4*)trow + e0 / kVec) : neg_inf_vec<DT>();
                wd[h] = e0 < V ? ld16((const uint4*)drow + e0 / kVec) : neg_inf_vec<DT>();
            }
#pragma unroll
            for (int h = 0; h < kH; ++h) {
#pragma unroll 1
                for (int q = 0; q < 4; ++q) {
                    const uint32_t a = q == 0 ? wt[h].x : q == 1 ? wt[h].y : q == 2 ? wt[h].z : wt[h].w;
                    const uint32_t b = q == 0 ? wd[h].x : q == 1 ? wd[h].y : q == 2 ? wd[h].z : wd[h].w;
                    if constexpr (DT == kBF16) {
                        f(bf16_lo(a), bf16_lo(b));
                        f(bf16_hi(a), bf16_hi(b));
                    } else {
                        f(__uint_as_float(a), __uint_as_float(b));
                    }
                }
            }
        } else {
            const int e0 = t * kTile + (lane + 64 * u0) * kVec;
#pragma unroll 1
            for (int e = e0; e < e0 + kVec; ++e) {
                const bool in = e < V;
                f(in ? load_elem<DT>(trow, e) : -INFINITY, in ? load_elem<DT>(drow, e) : -INFINITY);
            }
        }
    };
    // the same elements kHL vectors of each row at a time (the cold log2 pass,
    // whose element math is longest: more in flight does not fit the registers)
    constexpr int kHL = (ALIGNED && DT == kF32) ? 2 : 1;  // 8 elements of each row
    auto visit_log = [&](int t, int u0, auto&& f) {
        if constexpr (ALIGNED) {
            uint4 wt[kHL], wd[kHL];
#pragma unroll
            for (int h = 0; h < kHL; ++h) {
                const int e0 = t * kTile + (lane + 64 * (u0 + h)) * kVec;
                wt[h] = e0 < V ? ld16((const uint4*)trow + e0 / kVec) : neg_inf_vec<DT>();
                wd[h] = e0 < V ? ld16((const uint4*)drow + e0 / kVec) : neg_inf_vec<DT>();
            }
#pragma unroll
            for (int h = 0; h < kHL; ++h) {
#pragma unroll 1
                for (int q = 0; q < 4; ++q) {
                    const uint32_t a = q == 0 ? wt[h].x : q == 1 ? wt[h].y : q == 2 ? wt[h].z : wt[h].w;
                    const uint32_t b = q == 0 ? wd[h].x : q == 1 ? wd[h].y : q == 2 ? wd[h].z : wd[h].w;
                    if constexpr (DT == kBF16) {
                        f(bf16_lo(a), bf16_lo(b));
                        f(bf16_hi(a), bf16_hi(b));
                    } else {
                        f(__uint_as_float(a), __uint_as_float(b));
                    }
                }
            }
        } else {
            visit(t, u0, f);
        }
    };
    // the shift, and the largest relative target logit of the tokens the rows
    // share, of those where the target's exceeds the draft's, and of the others
    float sl = -INFINITY, m_sh = -INFINITY, m_tf = -INFINITY, m_df = -INFINITY;
    float g_df = INFINITY;  // the smallest ad - at where the draft's exceeds the target's
    for (int t = w; t < NT; t += kWaves)
        for (int u0 = 0; u0 < kU; u0 += kH)
            visit(t, u0, [&](float zt, float zd) {
                const float at = near_rel(zt, m_t), ad = near_rel(zd, m_d);
                if (at != ad) sl = fmaxf(sl, fmaxf(at, ad));
                // one update per maximum, no branch between them
                m_sh = fmaxf(m_sh, at == ad ? at : -INFINITY);
                m_tf = fmaxf(m_tf, ad < at ? at : -INFINITY);
                m_df = fmaxf(m_df, ad > at ? at : -INFINITY);
                g_df = fminf(g_df, ad > at ? ad - at : INFINITY);
            });
    sl = block_max_f_all(sl);
    double msh = (double)m_sh, mtf = (double)m_tf, mdf = (double)m_df, ngdf = -(double)g_df;
    block_max2_d_all(msh, mtf);
    block_max2_d_all(mdf, ngdf);
    double X = 0.0, D = 0.0, Y = 0.0, unused = 0.0;
    for (int t = w; t < NT; t += kWaves) {
        float sx = 0.f, sd = 0.f, sy = 0.f;
        for (int u0 = 0; u0 < kU; u0 += kH)
            visit(t, u0, [&](float zt, float zd) {
                const NearTerm tm = near_term(m_t, m_d, sl, c, zt, zd);  // absent elements: terms 0
                sx += tm.A;
                sd += tm.Dl;
                sy += tm.Bs;
            });
        X += (double)wave_sum(sx);
        D += (double)wave_sum(sd);
        Y += (double)wave_sum(sy);
    }
    if (lane != 0) X = D = Y = 0.0;  // every lane of a wave holds the wave's sums
    block_sum2_all(X, D);
    block_sum2_all(Y, unused);
    const double rho = X > 0.0 ? D / X : 0.0;
    const double sig = sl > -INFINITY ? (double)sl * (double)c : 0.0;  // the shift, log2 units
    const double scale = sl > -INFINITY ? exp2(sig) : 0.0;              // 2^(sl c), binary64
    // kappa in units of 2^(sl c): carried by a tree walk (after two or more
    // rejections at a node), else rho - mu 2^(-sl c) (mu = 0 after one rejection)
    double kappa;
    if (d.skap != 0) {
        kappa = desc_kappa(d, sig);
    } else {
        const double lmu = desc_lmu(d);
        double mus = 0.0;  // mu 2^(-sl c)
        if (lmu > -INFINITY) mus = sl > -INFINITY ? exp2(lmu - sig) : (double)FLT_MAX;
        kappa = rho - mus;
    }
    const double lam = 1.0 + desc_mu(d);
    const float kappa_f = (float)fmin(fmax(kappa, -(double)FLT_MAX), (double)FLT_MAX), lam_f = (float)lam;
    *ws = WSpec{kWResNear, c, m_t, m_d, lam_f, kappa_f, sl, 0.f, 0.f};
    const double Sd = X * (1.0 + rho * scale);  // the draft row's sum in A's units
    // kappa as sign and log2 (a carried kappa without forming 2^(lkap - sl c))
    int ks;
    double lk;
    if (d.skap != 0) {
        ks = d.lkap == -INFINITY ? 0 : d.skap;
        lk = d.lkap - sig;
    } else {
        ks = kappa > 0.0 ? 1 : kappa < 0.0 ? -1 : 0;
        lk = kappa != 0.0 ? log2(fabs(kappa)) : -INFINITY;
    }
    // binary32 terms in units of 2^(sl c) may lose every weight that decides the
    // draw (their total far below 1), or, for a round, the comparison of kappa Y
    // with W (both far below 1): then the weights are formed from their log2
    // (near_log_weight()), scaled by 2^-E with E the largest tile's log2 sum
    // rounded down.
    // Bounds of the largest weights from the maxima above say so in advance
    // where they can (the binary32 pass is then skipped); else the binary32
    // sums say so afterwards.
    const double llam = log2(lam), lV = log2((double)V);
    const double lky = (ks > 0 && Y > 0.0) ? lk + sig + log2(Y) : -INFINITY;  // log2 (kappa Y), units of 2^(sl c)
    const double e_sh = ks > 0 ? lk + msh * (double)c : -INFINITY;
    const double e_tf = llam + mtf * (double)c - sig + 1.0;
    // a token where the draft's logit exceeds the target's by x >= 1 has a
    // positive weight only if log2 |kappa| + sl c - log2 lam > x - 1 (near_log_bound())
    const double xg = -ngdf * (double)c;
    const bool df_zero = xg >= 1.0 && xg - 1.0 >= lk + sig - llam;
    const double e_df = (ks > 0 && !df_zero) ? lk + mdf * (double)c : -INFINITY;
    const bool pred_log = fmax(e_sh, fmax(e_tf, e_df)) + lV < -100.0 ||
                          (need_next && ks > 0 && !(lky > -90.0) && fmax(e_tf, e_df) + lV < -90.0);
    double zsum = 0.0, wdsum = 0.0;
    if (!pred_log) {
        for (int t = w; t < NT; t += kWaves) {
            float sw = 0.f, swd = 0.f;
            for (int u0 = 0; u0 < kU; u0 += kH)
                visit(t, u0, [&](float zt, float zd) {
                    const float wt = near_weight(m_t, m_d, sl, c, kappa_f, lam_f, zt, zd);
                    sw += wt;
                    if (near_rel(zt, m_t) != near_rel(zd, m_d)) swd += wt;
                });
            sw = wave_sum(sw);
            swd = wave_sum(swd);
            if (lane == 0) {
                s_w[t] = (double)sw;
                zsum += (double)sw;
                wdsum += (double)swd;
            }
        }
        block_sum2_all(zsum, wdsum);
    }
    double lz = zsum > 0.0 ? log2(zsum) : -INFINITY, lwd = wdsum > 0.0 ? log2(wdsum) : -INFINITY;
    const bool log_draw = pred_log || !(zsum > 0x1p-100);
    const bool log_w = pred_log || (need_next && !(wdsum > 0x1p-90) && ks > 0 && !(lky > -90.0));
    if (log_draw || log_w) {
        WSpec wl{kWResNearLog, c, m_t, m_d, lam_f, 0.f, sl, 0.f, 0.f, ks, lk, sig, 0.0};
        const float lkf = (float)fmax(lk, -3e38), sgf = (float)sig, llf = (float)llam;
        // one pass: each lane keeps a running largest log2 weight and the sum of
        // its weights scaled to it, for the tile (all tokens) and for the
        // differing tokens (all its tiles); a weight whose bound lies 64 below
        // the wave's largest so far adds less than 2^-63 of it and is left out.
        // For the draw each tile's log2 sum goes to s_w[t] first (else s_w keeps
        // the binary32 pass's tile weights).
        // the running maxima are binary32 (reference points only: every difference
        // to them is formed in binary64)
        float mw = -INFINITY;  // the differing tokens (W)
        float sw_d = 0.f;
        for (int t = w; t < NT; t += kWaves) {
            float mt = -INFINITY;
            float st = 0.f;
            // the wave's largest so far (one threshold for the whole wave, so
            // that the long element math runs only where some lane needs it)
            float thr = -INFINITY;
            for (int u0 = 0; u0 < kU; u0 += kHL) {
                visit_log(t, u0, [&](float zt, float zd) {
                    if (!(near_log_bound(ks, lkf, sgf, llf, c, m_t, m_d, zt, zd) >= thr)) return;
                    const double lw = near_log_weight(wl, zt, zd);
                    if (lw == -INFINITY) return;
                    if (lw > (double)mt) {
                        const float nm = (float)lw;
                        st *= exp2_fast((float)((double)mt - (double)nm));
                        mt = nm;
                    }
                    st += exp2_fast((float)(lw - (double)mt));
                    if (near_rel(zt, m_t) != near_rel(zd, m_d)) {
                        if (lw > (double)mw) {
                            const float nm = (float)lw;
                            sw_d *= exp2_fast((float)((double)mw - (double)nm));
                            mw = nm;
                        }
                        sw_d += exp2_fast((float)(lw - (double)mw));
                    }
                });
                float th = fminf(mt, mw);
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) th = fmaxf(th, __shfl_xor(th, off, 64));
                thr = fmaxf(thr, th - 64.f);
            }
            // the tile's log2 sum over the wave
            float M = mt;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
            const float S = wave_sum(M > -INFINITY && mt > -INFINITY ? st * exp2_fast((float)((double)mt - (double)M)) : 0.f);
            if (log_draw && lane == 0) s_w[t] = S > 0.f ? (double)M + log2((double)S) : -INFINITY;
        }
        // W over the workgroup (per-lane values into the block sum)
        double Mw = (double)mw, unused_w = -INFINITY;
        block_max2_d_all(Mw, unused_w);  // also orders the s_w writes above before the reads below
        double wdl = (Mw > -INFINITY && mw > -INFINITY) ? (double)sw_d * exp2((double)mw - Mw) : 0.0, unused_s = 0.0;
        block_sum2_all(wdl, unused_s);
        lwd = wdl > 0.0 ? Mw + log2(wdl) : -INFINITY;
        if (log_draw) {
            // the draw's scale E: the largest tile's log2 sum, rounded down
            double E = -INFINITY;
            for (int t = threadIdx.x; t < NT; t += kThreads) E = fmax(E, s_w[t]);
            double unused_e = -INFINITY;
            block_max2_d_all(E, unused_e);
            E = E > -INFINITY ? floor(E) : 0.0;
            wl.E = E;
            double zl = 0.0;
            for (int t = threadIdx.x; t < NT; t += kThreads) {
                const double v = s_w[t] > -INFINITY ? exp2(s_w[t] - E) : 0.0;
                s_w[t] = v;
                zl += v;
            }
            block_sum2_all(zl, unused_s);
            *ws = wl;
            zsum = zl;
            lz = zl > 0.0 ? E + log2(zl) : -INFINITY;
        }
    }
    pl->Z = zsum;
    pl->sq = Sd;
    pl->kappa = kappa;
    pl->lam = lam;
    pl->sh = sl > -INFINITY ? exp2(-sig) : 1.0;
    pl->exact = true;
    pl->lmass = (X > 0.0 && lz > -INFINITY) ? sig + lz - log2(Sd) : -INFINITY;
    pl->mass = pl->lmass > -INFINITY ? exp2(pl->lmass) : 0.0;
    pl->yd = Y;
    pl->lwd = lwd;
    pl->lu = sig;
    pl->lk = lk;
    pl->ks = ks;
}

// The residual draw's set-up in the deciding workgroup, from the far-form tile
// sums v[r][*] of tiles tid + r kThreads, for the residual max(0, p - lq q) with
// lam = 1 + mu (mu from d.mu): the tile weights into
// s_w[NT], the element weighting into *ws, the rest into *pl (with no residual
// mass left, s_w holds the target's own tile masses and *ws weighs by the
// target).  need_next: a tree walk's round, which also needs kappa after the
// next rejection (next_kappa()), so the chunks' near form is trusted only where
// its sums over the differing tokens lie far inside the binary32 range.
template <int DT, bool ALIGNED, int TPT>
__device__ __forceinline__ void plan_residual(const float (&v)[TPT][kDrawSums], int NT, const DrawDesc& d, const void* trow,
                              const void* drow, int V, double* s_w, WSpec* ws, ResidPlan* pl, bool need_next) {
    const int tid = threadIdx.x;
    const double lq = 1.0 + desc_mu(d);  // lam
    double sp = 0.0, sq = 0.0;           // far form: sum P, sum Q; near form: sum A, sum Dl
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
        sp += (double)v[r][kSumP];
        sq += (double)v[r][kSumQ];
    }
    block_sum2_all(sp, sq);
    double zr = 0.0, zp = 0.0;
    bool exact = false;  // the near form by this workgroup alone
    if (d.kind == kDrawResidualNear) {
        // the chunks' near-form sums (near_lin()): kappa carried by a tree walk,
        // else sum Dl / sum A - mu
        const NearLin nl = near_lin(d);
        const double kappa = d.skap != 0 ? desc_kappa(d, 0.0) : sp > 0.0 ? sq / sp - desc_mu(d) : 0.0;
        const double dk = kappa - (double)nl.kappa0;
        double yd = 0.0, wd = 0.0;
#pragma unroll
        for (int r = 0; r < TPT; ++r) {
            const int i = tid + r * kThreads;
            if (i < NT) {
                double w = (double)v[r][kSumW] + dk * (double)v[r][kSumG];
                w = w > 0.0 ? w : 0.0;
                s_w[i] = w;
                zr += w;
                zp += (double)v[r][kSumA];
                yd += (double)v[r][kSumY];
                wd += (double)v[r][kSumWd];
            }
        }
        block_sum2_all(zr, zp);
        block_sum2_all(yd, wd);
        // trusted when the tokens the rows share (crossing at kappa = 0) lie on
        // one side of both kappa0 and kappa with room to spare, and the mass is
        // far above what binary32 terms without a shift can carry (for a round,
        // the differing tokens' draft mass and kappa times it too)
        bool ok = sp > 0.0 && kappa * (double)nl.kappa0 > 0.0 && fabs(kappa) > 4.0 * fabs(dk) &&
                  zr > 0x1p-60 * sp;
        if (need_next) ok = ok && yd > 0x1p-80 * sp && (kappa <= 0.0 || kappa * yd > 0x1p-80 * sp);
        if (ok) {
            *ws = WSpec{kWResNear, d.c, d.m_t, d.m_d, nl.lam, (float)kappa, 0.f, 0.f, 0.f};
            const double Sd = sp + sq;  // S_d = sum B = sum A + sum Dl
            *pl = ResidPlan{zr,    zr / Sd, log2(zr / Sd), Sd, kappa, (double)nl.lam, 1.0, false, yd,
                            wd > 0.0 ? log2(wd) : -INFINITY, 0.0, kappa != 0.0 ? log2(fabs(kappa)) : -INFINITY,
                            kappa > 0.0 ? 1 : -1};
        } else {
            exact = true;
        }
    } else {
        const double Lam = sq > 0.0 ? lq * (sp / sq) : 0.0;  // lam S_t / S_d from the same terms
        const double Lam0 = lq * exp2((double)d.lq);
#pragma unroll
        for (int r = 0; r < TPT; ++r) {
            const int i = tid + r * kThreads;
            if (i < NT) {
                double w = (double)v[r][kSumW] - (Lam - Lam0) * (double)v[r][kSumG];
                w = w > 0.0 ? w : 0.0;
                s_w[i] = w;
                zr += w;
                zp += (double)v[r][kSumP];
            }
        }
        block_sum2_all(zr, zp);
        *ws = WSpec{kWResFar, d.c, d.m_t, d.m_d, (float)Lam, 0.f, 0.f, neg_scaled(d.m_t, d.c), neg_scaled(d.m_d, d.c)};
        *pl = ResidPlan{zr, sp > 0.0 ? zr / sp : 0.0, (sp > 0.0 && zr > 0.0) ? log2(zr / sp) : -INFINITY, sq, 0.0, 0.0,
                        1.0, false, 0.0, -INFINITY, 0.0, -INFINITY, 0};
        exact = sq > 0.0 && zr < kNearZ * sp;  // a small residual after all
    }
    if (exact) {
        __syncthreads();
        near_exact_tiles<DT, ALIGNED>(trow, drow, V, NT, d, s_w, ws, pl, need_next);
        zr = pl->Z;
    }
    if (!(zr > 0.0)) {
        // no residual mass left after rounding: draw from p_k
        __syncthreads();
#pragma unroll
        for (int r = 0; r < TPT; ++r) {
            const int i = tid + r * kThreads;
            if (i < NT) s_w[i] = (double)v[r][kSumP];
        }
        // (the chunks' sum P is in the near form's units 2^((z - m_t) c), else in
        // the far form's)
        *ws = d.kind == kDrawResidualNear ? target_spec(d) : target_p_spec(d);
        *pl = ResidPlan{-zp, 0.0, -INFINITY, 0.0, 0.0, 0.0, 1.0, false, 0.0, -INFINITY, 0.0, -INFINITY, 0};
    }
    __syncthreads();
}

// The acceptance ratio (p(x) - lam q(x)) / (M q(x)) of a token with logits zt,
// zd under the residual that plan_residual() formed (M its mass; 0 when it has
// none), in binary64 from the plan's own terms:
//   far form:  p - lam q = (P - Lam Q) / sum P, M = Z / sum P, q = Q / sum Q;
//   near form: p - lam q = 2^(sl c) w / S_d, M = 2^(sl c) Z / S_d, q = B / S_d
//              (w = kappa A - lam Dl of near_term());
// both give w sq / (Z q') with q' = Q or B.  q(x) = 0 < p(x) - lam q(x): +inf.
__device__ __forceinline__ double resid_ratio(const WSpec& ws, const ResidPlan& pl, float zt, float zd) {
    if (!(pl.Z > 0.0) || target_only(ws)) return 0.0;
    if (ws.mode == kWResNearLog) {
        // w S_d / (Z B) from the log2 weight: Z = 2^E sum in units of 2^(sl c)
        const float ad = near_rel(zd, ws.m_d);
        if (ad == -INFINITY) return near_rel(zt, ws.mA) == -INFINITY ? 0.0 : INFINITY;  // q(x) = 0
        const double lw = near_log_weight(ws, zt, zd);
        if (lw == -INFINITY) return 0.0;
        return exp2(lw - (ws.E + log2(pl.Z)) + log2(pl.sq) - (double)ad * (double)ws.c);
    }
    if (ws.mode == kWResFar) {
        // (P - Lam Q) sq / (Z Q) = (P / Q - Lam) sq / Z, with P / Q from the exponents in
        // binary64, so that the ratio keeps its value where P and Q lie below the
        // binary32 range (a token far below both rows' maxima at low T)
        if (zt == -INFINITY) return 0.0;       // p(x) = 0
        if (zd == -INFINITY) return INFINITY;  // q(x) = 0 < p(x)
        const double c = (double)ws.c;
        const double lpq = ((double)zt * c + (double)ws.nmt) - ((double)zd * c + (double)ws.nmd);
        const double v = exp2(lpq) - (double)ws.lam;
        return v > 0.0 ? v * pl.sq / pl.Z : 0.0;
    }
    // near form: w / B with r = A / B = 2^((at - ad) c): w / B = kappa r - lam (1 - r) 2^(-sl c)
    // (a token the rows share has r = 1 and no second term)
    const float at = near_rel(zt, ws.mA), ad = near_rel(zd, ws.m_d);
    if (ad == -INFINITY) return at == -INFINITY ? 0.0 : INFINITY;  // q(x) = 0
    if (at == -INFINITY) return 0.0;                                  // p(x) = 0 < q(x)
    double wb = pl.kappa;
    if (at != ad) {
        // 1 - r in binary64 keeps about 16 - log10(1 / |xr|) digits, and two
        // distinct binary32 relative logits give |xr| far above 1e-8
        const double xr = ((double)at - (double)ad) * (double)ws.c;
        const double r = exp2(xr), sh = pl.sh;  // sh = 2^(-sl c) >= 1
        if (!(r < INFINITY)) return pl.kappa + pl.lam * sh > 0.0 ? INFINITY : 0.0;  // w / B = r (kappa + lam sh) - lam sh
        wb = pl.kappa * r - pl.lam * (1.0 - r) * sh;
    }
    return wb > 0.0 ? wb * pl.sq / pl.Z : 0.0;
}

// One chunk of a residual reduction of the pair (trow, drow) (drow unused when
// !has_draft: the target row alone): its tiles [c kDrawTiles, ...) loaded once
// (wave w owns kDrawTiles / kWaves whole tiles, lane l reads vectors l, l + 64,
// ... of each, all loads issued before the first use), the far-form tile sums
// at lam0 = (1 + mu) 2^d.lq, or for a kDrawResidualNear draw the near form's
// (near_lin()), handed over by atomic exchange into dsum[q][tile], completed
// before the function returns.
template <int DT, bool ALIGNED>
__device__ __forceinline__ void residual_chunk(const void* trow, const void* drow, bool has_draft, const DrawDesc& d,
                                               int V, int NT, int c, unsigned* dsum) {
    constexpr int kVec = Elem<DT>::kVec;
    constexpr int kTile = kThreads * kVec;
    constexpr int kTilesPerWave = kDrawTiles / kWaves;
    constexpr int kU = kThreads / 64;  // vectors per lane per tile
    static_assert(kDrawTiles % kWaves == 0, "draw chunk must split evenly over the waves");
    const float lam0 = (float)(1.0 + desc_mu(d)) * exp2_fast(d.lq);
    const float nmt = neg_scaled(d.m_t, d.c), nmd = neg_scaled(d.m_d, d.c);
    const int tile0 = c * kDrawTiles;
    const int cnt = min(kDrawTiles, NT - tile0);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    // vector u of tile i of this wave (raw 16-byte vectors: bf16 pairs or fp32)
    auto load = [&](int i, int u, uint4& vt, uint4& vd) {
        const int e0 = (tile0 + wv * kTilesPerWave + i) * kTile + (lane + 64 * u) * kVec;
        const bool ok = wv * kTilesPerWave + i < cnt && e0 < V;
        if constexpr (ALIGNED) {
            vt = ok ? ld16((const uint4*)trow + e0 / kVec) : neg_inf_vec<DT>();
            vd = (ok && has_draft) ? ld16((const uint4*)drow + e0 / kVec) : neg_inf_vec<DT>();
        } else {
            vt = load_raw<DT>(trow, e0, ok ? V : 0);
            vd = load_raw<DT>(drow, e0, (ok && has_draft) ? V : 0);
        }
    };
    unsigned dep = 0u;
    auto hand_over = [&](int i, FarSums fs) {
        fs = wave_far_sums(fs);
        const int t = wv * kTilesPerWave + i;
        if (lane < 4 && t < cnt) dep ^= xchg32(dsum + (size_t)lane * NT + tile0 + t, __float_as_uint(far_sum_at(fs, lane)));
    };
    auto hand_over_near = [&](int i, NearSums ns) {
        ns = wave_near_sums(ns);
        const int t = wv * kTilesPerWave + i;
        if (lane < kDrawSums && t < cnt)
            dep ^= xchg32(dsum + (size_t)lane * NT + tile0 + t, __float_as_uint(near_sum_at(ns, lane)));
    };
    if (d.kind == kDrawResidualNear) {
        // the near form's sums (near_lin()), every vector of the chunk in flight
        // before the first use; the element math is long, so four elements of
        // each row at a time (unrolled over a whole vector it spills)
        const NearLin nl = near_lin(d);
        uint4 rt[kTilesPerWave][kU], rd[kTilesPerWave][kU];
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i)
#pragma unroll
            for (int u = 0; u < kU; ++u) load(i, u, rt[i][u], rd[i][u]);
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i) {
            NearSums fs{0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // absent elements read -inf on both rows: every term is 0
#pragma unroll
            for (int u = 0; u < kU; ++u) {
#pragma unroll 4
                for (int e = 0; e < kVec; ++e) {
                    const int q = DT == kBF16 ? e >> 1 : e;
                    const uint4 vt = rt[i][u], vd = rd[i][u];
                    const uint32_t a = q == 0 ? vt.x : q == 1 ? vt.y : q == 2 ? vt.z : vt.w;
                    const uint32_t bb = q == 0 ? vd.x : q == 1 ? vd.y : q == 2 ? vd.z : vd.w;
                    if constexpr (DT == kBF16) {
                        const bool hi = e & 1;
                        near_accum(fs, d, nl, hi ? bf16_hi(a) : bf16_lo(a), hi ? bf16_hi(bb) : bf16_lo(bb));
                    } else {
                        near_accum(fs, d, nl, __uint_as_float(a), __uint_as_float(bb));
                    }
                }
            }
            hand_over_near(i, fs);
        }
    } else {
        // the far form's sums, every vector of the chunk in flight before the first use
        uint4 rt[kTilesPerWave][kU], rd[kTilesPerWave][kU];
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i)
#pragma unroll
            for (int u = 0; u < kU; ++u) load(i, u, rt[i][u], rd[i][u]);
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i) {
            FarSums fs{0.f, 0.f, 0.f, 0.f};  // absent elements read -inf on both rows: every term is 0
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                float zt[kVec], zd[kVec];
                unpack<DT>(rt[i][u], zt);
                unpack<DT>(rd[i][u], zd);
#pragma unroll
                for (int e = 0; e < kVec; ++e) far_accum(fs, nmt, nmd, d.c, lam0, zt[e], zd[e]);
            }
            hand_over(i, fs);
        }
    }
    // this wave's exchanges have been performed before the workgroup arrives
    asm volatile("" ::"v"(dep));
    __builtin_amdgcn_s_waitcnt(0);
}

constexpr int kTPT = kMaxTiles / kThreads;  // tiles per thread, at most, in the deciding workgroup

// The deciding workgroup collects (and resets to zero) the tile sums of the whole
// row pair: v[r][q] = sum q of tile tid + r kThreads, the first nq sums (the far
// form hands over 4, the near form kDrawSums; the rest read 0).
__device__ __forceinline__ void collect_tile_sums(float (&v)[kTPT][kDrawSums], int NT, unsigned* dsum, int nq) {
#pragma unroll
    for (int r = 0; r < kTPT; ++r) {
        const int i = threadIdx.x + r * kThreads;
#pragma unroll
        for (int q = 0; q < kDrawSums; ++q)
            v[r][q] = (i < NT && q < nq) ? __uint_as_float(xchg32(dsum + (size_t)q * NT + i, 0u)) : 0.f;
    }
}

template <int DT, bool ALIGNED>
__device__ __forceinline__ void draw_item(const DrawParams& p, int b, int c, double* s_buf) {
    const DrawDesc d = p.desc[b];
    if (d.kind == kDrawNone) return;
    const int n = p.n, V = p.V, NT = p.NT, tid = threadIdx.x;
    const void* trow = row_ptr<DT>(p.target, target_row_of(p.R, p.row_index, b, d.k), V);
    if (d.kind == kDrawBonus) {
        if (c != 0) return;
        const int y = tile_draw<DT, ALIGNED, false>(p.tiles + (size_t)b * NT, NT, V, d, trow, s_buf);
        for (int i = tid; i < NT; i += kThreads) p.tiles[(size_t)b * NT + i] = 0ull;  // used: leave zero
        if (tid == 0) {
            p.emitted[(size_t)b * (n + 1) + d.slot] = y;
            if (p.mtp_tokens) p.mtp_tokens[(size_t)b * (n + 1) + d.slot] = y;
            p.desc[b] = DrawDesc{};
        }
        return;
    }
    // kDrawTarget: the whole of target row k alone (no draft row: Q = 0, W = P)
    const bool has_draft = is_residual_draw(d.kind);
    const void* drow = has_draft ? row_ptr<DT>(p.draft, (long long)b * n + d.k, V) : nullptr;
    unsigned* dsum = reinterpret_cast<unsigned*>(p.dsum) + (size_t)b * kDrawSums * NT;
    residual_chunk<DT, ALIGNED>(trow, drow, has_draft, d, V, NT, c, dsum);
    __syncthreads();
    __shared__ int s_last;
    if (tid == 0) s_last = (arrive(&p.cnt[b], 0ull) == (unsigned)p.NCd - 1u);
    __syncthreads();
    if (!s_last) return;

    // last workgroup: collect (and reset) the per-tile sums of the whole row pair
    float v[kTPT][kDrawSums];
    collect_tile_sums(v, NT, dsum, d.kind == kDrawResidualNear ? kDrawSums : 4);
    WSpec ws;
    ResidPlan pl;
    plan_residual<DT, ALIGNED, kTPT>(v, NT, d, trow, drow, V, s_buf, &ws, &pl, false);
    const double Z = pl.Z;
    if (!has_draft) ws = target_p_spec(d);  // weights P: the target row's own distribution, in its tile sums' units
    if (Z <= 0.0 && tid == 0 && p.flags) atomicOr(p.flags, (uint32_t)SV_FLAG_ZERO_RESIDUAL);
    const double t = (double)d.u * fabs(Z);
    const Pick pk = block_first_crossing(NT, t, [&](int i) { return s_buf[i]; });
    int tile = pk.i;
    bool take_last = false;
    if (tile < 0) {  // t at or past the total through rounding: the last tile with mass
        int my_last = -1;
        for (int i = tid; i < NT; i += kThreads)
            if (s_buf[i] > 0.0) my_last = i;
        const int lt = block_max_all(my_last);
        tile = lt < 0 ? 0 : lt;
        take_last = true;
    }
    const int y = scan_tile<DT, ALIGNED>(ws, trow, drow, V, tile, pk.before, t, take_last);
    // row L's tile partials (written by the stats pass, unused here): leave them zero
    for (int i = tid; i < NT; i += kThreads) p.tiles[(size_t)b * NT + i] = 0ull;
    if (tid == 0) {
        p.emitted[(size_t)b * (n + 1) + d.slot] = y;
        if (p.mtp_tokens) p.mtp_tokens[(size_t)b * (n + 1) + d.slot] = y;
        p.desc[b] = DrawDesc{};
        xchg32(&p.cnt[b], 0u);
    }
}

// kappa_{k+1} = kappa_k - M_k from the residual the round formed at lam_k.  The
// near form has the sums over the tokens whose relative logits differ, Y = sum B
// and W = sum max(0, kappa_k A - lam_k Dl), while the tokens the rows share
// contribute max(0, kappa_k) times their own sum to M_k S_d and their sum is
// S_d - Y, so
//   kappa_{k+1} = (kappa_k Y - W) / S_d  (kappa_k > 0),  kappa_k - W / S_d  (else):
// no difference of nearly equal numbers is formed unless kappa_k Y and W are
// themselves that close.  The far form (mass above the near form's threshold,
// where the difference keeps its digits) and a residual with no mass left
// (M_k = 0) take kappa_k - M_k in binary64.
__device__ __forceinline__ SLog2 next_kappa(const DrawDesc& d, const WSpec& ws, const ResidPlan& pl, double St,
                                           double Sd) {
    if ((ws.mode == kWResNear || ws.mode == kWResNearLog) && pl.Z > 0.0) {
        SLog2 r;
        if (pl.ks > 0) {
            const SLog2 ky{1, pl.yd > 0.0 ? pl.lk + pl.lu + log2(pl.yd) : -INFINITY};
            r = slog2_add(ky, SLog2{-1, pl.lwd});
        } else {
            // -(|kappa_k| S_d + W)
            r = SLog2{-1, log2_add(pl.ks != 0 ? pl.lk + log2(pl.sq) : -INFINITY, pl.lwd)};
        }
        if (r.l == -INFINITY) return SLog2{1, -INFINITY};
        return SLog2{r.s, r.l + pl.lu - log2(pl.sq)};
    }
    const double kk = d.skap != 0 ? desc_kappa(d, 0.0) : Sd / St - 1.0;
    const double M = (!target_only(ws) && pl.Z > 0.0) ? exp2(pl.lmass) : 0.0;
    return slog2_of(kk - M);
}

// One round of the sampling tree walks, workgroup (b, c): if sequence b's walk
// is pending at node u with lam, chunk c of the residual reduction of the pair
// (target row u, draft row u); the last workgroup forms M = sum max(0, p_u -
// lam q_u) (plan_residual: exact ratio, near form when small) and runs the walk
// on: it finishes (outputs, draw descriptor; its state cleared) or stops
// pending again for the next round.
template <int DT, bool ALIGNED>
__device__ __forceinline__ void round_item(const RoundParams& p, int b, int c, double* s_buf) {
    const TreeWalk* gw = p.walk + b;
    if (gw->status != kWalkPending) return;
    const int n = p.n, V = p.V, NT = p.NT, tid = threadIdx.x;
    const int u = gw->u;
    const TreeRowsLayout lay = tree_rows_layout(n);
    char* rows = p.trows + (size_t)b * lay.stride;
    const float* gmt = reinterpret_cast<const float*>(rows + lay.mt);
    const double* gSt = reinterpret_cast<const double*>(rows + lay.St);
    const float* gmd = reinterpret_cast<const float*>(rows + lay.md);
    const double* gSd = reinterpret_cast<const double*>(rows + lay.Sd);
    DrawDesc d{};
    d.kind = gw->zb < kNearZ ? kDrawResidualNear : kDrawResidual;
    d.k = u;
    d.c = gw->c;
    d.m_t = gmt[u];
    d.m_d = gmd[u];
    d.lq = (float)log2(gSt[u] / gSd[u]);
    d.mu = encode_mu(gw->lmu);
    d.skap = gw->skap;
    d.lkap = gw->lkap;
    const void* trow = row_ptr<DT>(p.target, (long long)b * (n + 1) + u, V);
    const void* drow = row_ptr<DT>(p.draft, (long long)b * n + u, V);
    unsigned* dsum = reinterpret_cast<unsigned*>(p.dsum) + (size_t)b * kDrawSums * NT;
    residual_chunk<DT, ALIGNED>(trow, drow, true, d, V, NT, c, dsum);
    __syncthreads();
    __shared__ int s_last;
    if (tid == 0) s_last = (arrive(&p.cnt[b], 0ull) == (unsigned)p.NCd - 1u);
    __syncthreads();
    if (!s_last) return;

    float v[kTPT][kDrawSums];
    collect_tile_sums(v, NT, dsum, d.kind == kDrawResidualNear ? kDrawSums : 4);
    WSpec ws;
    ResidPlan pl;
    plan_residual<DT, ALIGNED, kTPT>(v, NT, d, trow, drow, V, s_buf, &ws, &pl, true);
    // the pending test: the walk's next child at u, under this residual (the
    // plan goes through LDS, so its registers are free for the ratio's binary64 math)
    __shared__ RoundStep s_step;
    __shared__ WSpec s_ws;
    __shared__ ResidPlan s_pl;
    if (tid == 0) {
        s_ws = ws;
        s_pl = pl;
    }
    if (tid == 0) {
        const SLog2 kn = next_kappa(d, s_ws, s_pl, gSt[u], gSd[u]);
        RoundStep st{0.0, s_pl.lmass, kn.l, kn.s};
        const int* par = p.parents + (size_t)b * n;
        const int L0 = min(max(p.lens[b], 0), n);
        for (int t = gw->next; t < L0; ++t)
            if (par[t] == u) {
                const int x = p.tokens[(size_t)b * n + t];
                if (x >= 0 && x < V)
                    st.ratio = resid_ratio(s_ws, s_pl, reinterpret_cast<const float*>(rows + lay.gt)[t],
                                           reinterpret_cast<const float*>(rows + lay.gd)[t]);
                break;
            }
        s_step = st;
    }
    // the walk's rows, staged in LDS
    __shared__ float s_mt[kMaxDraft + 1], s_md[kMaxDraft], s_gt[kMaxDraft], s_gd[kMaxDraft];
    __shared__ double s_St[kMaxDraft + 1], s_Sd[kMaxDraft];
    __shared__ int s_x[kMaxDraft], s_par[kMaxDraft];
    const int L = min(max(p.lens[b], 0), n);
    for (int i = tid; i <= L; i += kThreads) {
        s_mt[i] = gmt[i];
        s_St[i] = gSt[i];
    }
    for (int j = tid; j < L; j += kThreads) {
        s_md[j] = gmd[j];
        s_Sd[j] = gSd[j];
        s_gt[j] = reinterpret_cast<const float*>(rows + lay.gt)[j];
        s_gd[j] = reinterpret_cast<const float*>(rows + lay.gd)[j];
        s_x[j] = p.tokens[(size_t)b * n + j];
        const int par = p.parents[(size_t)b * n + j];
        s_par[j] = (par >= 0 && par <= j) ? par : -1;
    }
    __shared__ TreeWalk s_walk;  // the walk's state (LDS: its path is indexed at run time)
    __syncthreads();
    if (tid == 0) {
        const WalkRows r{s_mt, s_St, s_md, s_Sd, s_gt, s_gd, s_x, s_par};
        TreeWalk& w = s_walk;
        w = *gw;
        DrawDesc dd;
        const float* uni = p.unif + (size_t)b * (n + 1);
        const bool done = tree_walk_run(w, r, L, V, uni, p.can_pend != 0, s_step, true, &dd);
        if (done) tree_walk_finish(w, dd, s_x, n, uni[n], p.acc, p.emitted, p.path, p.desc, p.flags, b);
        tree_walk_store(w, !done, r, L, n, p.walk + b, rows);
        xchg32(&p.cnt[b], 0u);
    }
}

// One workgroup per (sequence, chunk), sequence-major.  The aligned kernel is
// held to 96 VGPRs (5 waves per SIMD; the near residual's five tile sums do not
// fit 80 without spilling); the element-wise unaligned one is left to the
// compiler.
template <int DT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(SV_DRAW_WPE))) void k_draw(DrawParams p) {
    __shared__ double s_buf[kMaxTiles];
    draw_item<DT, true>(p, blockIdx.x / p.NCd, blockIdx.x % p.NCd, s_buf);
}
template <int DT>
__global__ __launch_bounds__(kThreads) void k_draw_unaligned(DrawParams p) {
    __shared__ double s_buf[kMaxTiles];
    draw_item<DT, false>(p, blockIdx.x / p.NCd, blockIdx.x % p.NCd, s_buf);
}

// One round of the sampling tree walks (the draw pass's layout).
template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k_tree_round(RoundParams p) {
    __shared__ double s_buf[kMaxTiles];
    round_item<DT, ALIGNED>(p, blockIdx.x / p.NCd, blockIdx.x % p.NCd, s_buf);
}

// --------------------------------------------------------------- MTP shift / insert

template <bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k_mtp(MtpParams p) {
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long nthreads = (long long)gridDim.x * kThreads;
    if (gid < p.B) {
        // tokens: left shift by one in place (ascending, so each slot is read
        // before it is overwritten), then the target's next token at slot a
        const int n = p.n;
        int32_t* t = p.tokens + gid * (n + 1);
        shift_tokens(p.tokens, (int)gid, n);
        int a = p.acc[gid];
        a = a < 0 ? 0 : (a > n ? n : a);
        t[a] = p.emitted[gid * (n + 1) + a];
    }
    if (p.hsrc == nullptr || p.hdst == nullptr || p.hsrc == p.hdst) return;
    if constexpr (ALIGNED) {
        // hidden carry: each workgroup copies one contiguous region of
        // kThreads * SV_COPY_VECS 16-byte vectors, 4 loads in flight per thread
        const long long nvec = p.hidden_elems / 8;
        const u32x4* src = (const u32x4*)p.hsrc;
        u32x4* dst = (u32x4*)p.hdst;
        constexpr int kPer = kThreads * SV_COPY_VECS;
        for (long long base = (long long)blockIdx.x * kPer; base < nvec; base += (long long)gridDim.x * kPer)
            copy_range(src, dst, base, (base + kPer < nvec) ? base + kPer : nvec);
        // tail elements past the last full vector
        const long long tail0 = nvec * 8;
        const uint16_t* s16 = (const uint16_t*)p.hsrc;
        uint16_t* d16 = (uint16_t*)p.hdst;
        for (long long i = tail0 + gid; i < p.hidden_elems; i += nthreads) d16[i] = s16[i];
    } else {
        const uint16_t* s16 = (const uint16_t*)p.hsrc;
        uint16_t* d16 = (uint16_t*)p.hdst;
        for (long long i = gid; i < p.hidden_elems; i += nthreads) d16[i] = s16[i];
    }
}

// --------------------------------------------------------------- workspace clear

__global__ __launch_bounds__(kThreads) void k_clear(uint4* ws, long long nvec, uint8_t* tail, int ntail) {
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long nthreads = (long long)gridDim.x * kThreads;
    for (long long v = gid; v < nvec; v += nthreads) ws[v] = make_uint4(0, 0, 0, 0);
    if (gid < ntail) tail[gid] = 0;
}

// --------------------------------------------------------------- debug softmax

template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k_softmax_debug(const void* logits, const float* temp, int V,
                                                            float* out) {
    const int r = blockIdx.x;
    const float T = temp[r];
    const void* row = row_ptr<DT>(logits, r, V);
    float* o = out + (size_t)r * V;
    if (!(T > 0.f)) {
        for (int i = threadIdx.x; i < V; i += kThreads) o[i] = __builtin_nanf("");
        return;
    }
    const float c = exp2_scale(T);
    __shared__ MS s_ms;
    const MS ms = wg_softmax_tiles<DT, ALIGNED>(row, 0, V, c, nullptr);
    if (threadIdx.x == 0) s_ms = ms;
    __syncthreads();
    const float m = s_ms.m;
    const float inv_s = (float)(1.0 / (double)s_ms.s);
    for (int i = threadIdx.x; i < V; i += kThreads) o[i] = exp2_fast((load_elem<DT>(row, i) - m) * c) * inv_s;
}

// --------------------------------------------------------------- debug residual weights

// Parity/debug only: for row pair r (target row r, draft row r, temperature
// temp[r] > 0), the residual weights a draw after a rejection would scan, formed
// by the draw pass's own code: the descriptor's statistics from this kernel's
// own reduction of each row, the far-form tile sums as the draw chunks form them
// (wave w takes tiles w, w + kWaves, ..., lane l the same elements of a tile),
// the deciding workgroup's set-up (plan_residual(): the far form, or the near
// form when the residual mass is small), then every element's weight.
// Outputs: w_out[r][V] the element weights, tile_out[r][NT] (nullable) the
// tiles' weights the tile pick uses, info_out[r][4] (nullable) {0 far / 1 near from
// the chunks' sums / 2 near by one workgroup / 3 the same from log2 weights, lam
// (far form) or 0, kappa (near form) or 0, the residual mass}.
template <int DT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k_residual_debug(const void* target, const void* draft, const float* temp,
                                                             int V, int NT, float* w_out, double* tile_out,
                                                             float* info_out) {
    constexpr int kVec = Elem<DT>::kVec;
    constexpr int kTile = kThreads * kVec;
    constexpr int kU = kThreads / 64;
    constexpr int kTPT = kMaxTiles / kThreads;
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const void* trow = row_ptr<DT>(target, r, V);
    const void* drow = row_ptr<DT>(draft, r, V);
    const float T = temp[r];
    if (!(T > 0.f)) {
        for (int i = tid; i < V; i += kThreads) w_out[(size_t)r * V + i] = __builtin_nanf("");
        return;
    }
    const float c = exp2_scale(T);
    __shared__ MS s_t, s_d;
    const MS a = wg_softmax_tiles<DT, ALIGNED>(trow, 0, V, c, nullptr);
    if (tid == 0) s_t = a;
    __syncthreads();
    const MS bq = wg_softmax_tiles<DT, ALIGNED>(drow, 0, V, c, nullptr);
    if (tid == 0) s_d = bq;
    __syncthreads();
    DrawDesc d{};
    d.kind = kDrawResidual;
    d.c = c;
    d.m_t = s_t.m;
    d.m_d = s_d.m;
    d.lq = (float)log2((double)s_t.s / (double)s_d.s);
    const float lam0 = exp2_fast(d.lq);
    const float nmt = neg_scaled(d.m_t, c), nmd = neg_scaled(d.m_d, c);
    __shared__ float s_sum[kDrawSums][kMaxTiles];
    for (int t = w; t < NT; t += kWaves) {
        FarSums fs{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            float zt[kVec], zd[kVec];
            const int e0 = t * kTile + (lane + 64 * u) * kVec;
            load_vec<DT, ALIGNED>(trow, e0, V, zt);
            load_vec<DT, ALIGNED>(drow, e0, V, zd);
#pragma unroll
            for (int e = 0; e < kVec; ++e) far_accum(fs, nmt, nmd, c, lam0, zt[e], zd[e]);
        }
        fs = wave_far_sums(fs);
        if (lane < 4) s_sum[lane][t] = far_sum_at(fs, lane);
    }
    __syncthreads();
    // a residual mass below the near form's threshold: the tile sums a draw's
    // chunks hand over when the decision marks it (kDrawResidualNear)
    double zw = 0.0, zp = 0.0;
    for (int i = tid; i < NT; i += kThreads) {
        zw += (double)s_sum[kSumW][i];
        zp += (double)s_sum[kSumP][i];
    }
    block_sum2_all(zw, zp);
    if (zw < kNearZ * zp) {
        d.kind = kDrawResidualNear;
        const NearLin nl = near_lin(d);
        for (int t = w; t < NT; t += kWaves) {
            NearSums fs{0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int u = 0; u < kU; ++u) {
                float zt[kVec], zd[kVec];
                const int e0 = t * kTile + (lane + 64 * u) * kVec;
                load_vec<DT, ALIGNED>(trow, e0, V, zt);
                load_vec<DT, ALIGNED>(drow, e0, V, zd);
#pragma unroll 1
                for (int e = 0; e < kVec; ++e) near_accum(fs, d, nl, zt[e], zd[e]);
            }
            fs = wave_near_sums(fs);
            if (lane < kDrawSums) s_sum[lane][t] = near_sum_at(fs, lane);
        }
        __syncthreads();
    }
    float v[kTPT][kDrawSums];
    const int nq = d.kind == kDrawResidualNear ? kDrawSums : 4;
#pragma unroll
    for (int q = 0; q < kTPT; ++q) {
        const int i = tid + q * kThreads;
#pragma unroll
        for (int k = 0; k < kDrawSums; ++k) v[q][k] = (i < NT && k < nq) ? s_sum[k][i] : 0.f;
    }
    __shared__ double s_w[kMaxTiles];
    WSpec ws;
    ResidPlan pl;
    plan_residual<DT, ALIGNED, kTPT>(v, NT, d, trow, drow, V, s_w, &ws, &pl, false);
    const bool near = ws.mode == kWResNear || ws.mode == kWResNearLog;
    if (tile_out)
        for (int i = tid; i < NT; i += kThreads) tile_out[(size_t)r * NT + i] = s_w[i];
    for (int i = tid; i < V; i += kThreads)
        w_out[(size_t)r * V + i] = elem_weight(ws, load_elem<DT>(trow, i), load_elem<DT>(drow, i));
    if (info_out && tid == 0) {
        info_out[(size_t)r * 4 + 0] = ws.mode == kWResNearLog ? 3.f : near ? (pl.exact ? 2.f : 1.f) : 0.f;
        info_out[(size_t)r * 4 + 1] = ws.mode == kWResFar ? ws.lam : 0.f;
        info_out[(size_t)r * 4 + 2] = near ? ws.kappa : 0.f;
        info_out[(size_t)r * 4 + 3] = (float)pl.mass;
    }
}

hipError_t launch_residual_debug(const void* target, const void* draft, Dt dt, const float* temp, int rows, int V,
                                 int NT, float* w_out, double* tile_out, float* info_out, bool aligned,
                                 hipStream_t s) {
    const dim3 grid((unsigned)rows), block(kThreads);
#define SV_RD(DT_, AL_) \
    hipLaunchKernelGGL((k_residual_debug<DT_, AL_>), grid, block, 0, s, target, draft, temp, V, NT, w_out, tile_out, info_out)
    if (dt == kBF16) { if (aligned) SV_RD(kBF16, true); else SV_RD(kBF16, false); }
    else { if (aligned) SV_RD(kF32, true); else SV_RD(kF32, false); }
#undef SV_RD
    return hipGetLastError();
}

// --------------------------------------------------------------- launches

// Decision of greedy sequences whose row argmax keys another pass has already
// merged (one key per row at chunk slot 0, NC = 1): the fused logit projection.
// One workgroup per sequence.
__global__ __launch_bounds__(kThreads) void k_decide_greedy(StatsParams p) {
    const int b = blockIdx.x;
    decide<kBF16, kGreedy, true>(p, b, seq_info<kGreedy>(p, b));
}

hipError_t launch_decide_greedy(const StatsParams& p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    hipLaunchKernelGGL(k_decide_greedy, dim3((unsigned)p.B), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_stats(const StatsParams& p, Dt dt, Mode mode, bool aligned, hipStream_t s) {
    const unsigned blocks = (unsigned)((long long)p.B * p.S * p.NC);
    const dim3 grid(blocks), block(kThreads);
    if (mode == kSample && p.draw_in_stats) {
        if (dt == kBF16) {
            if (aligned) hipLaunchKernelGGL((k_stats_draw<kBF16, true>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((k_stats_draw<kBF16, false>), grid, block, 0, s, p);
        } else {
            if (aligned) hipLaunchKernelGGL((k_stats_draw<kF32, true>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((k_stats_draw<kF32, false>), grid, block, 0, s, p);
        }
        return hipGetLastError();
    }
#define SV_STATS(DT_, MODE_, AL_) hipLaunchKernelGGL((k_stats<DT_, MODE_, AL_>), grid, block, 0, s, p)
    if (dt == kBF16) {
        if (mode == kSample) { if (aligned) SV_STATS(kBF16, kSample, true); else SV_STATS(kBF16, kSample, false); }
        else { if (aligned) SV_STATS(kBF16, kGreedy, true); else SV_STATS(kBF16, kGreedy, false); }
    } else {
        if (mode == kSample) { if (aligned) SV_STATS(kF32, kSample, true); else SV_STATS(kF32, kSample, false); }
        else { if (aligned) SV_STATS(kF32, kGreedy, true); else SV_STATS(kF32, kGreedy, false); }
    }
#undef SV_STATS
    return hipGetLastError();
}

hipError_t launch_tree(const StatsParams& p, Dt dt, bool aligned, hipStream_t s) {
    const unsigned blocks = (unsigned)((long long)p.B * p.S * p.NC);
    const dim3 grid(blocks), block(kThreads);
    if (dt == kBF16) {
        if (aligned) hipLaunchKernelGGL((k_stats_tree<kBF16, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_stats_tree<kBF16, false>), grid, block, 0, s, p);
    } else {
        if (aligned) hipLaunchKernelGGL((k_stats_tree<kF32, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_stats_tree<kF32, false>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_tree_sample(const StatsParams& p, Dt dt, bool aligned, hipStream_t s) {
    const unsigned blocks = (unsigned)((long long)p.B * p.S * p.NC);
    const dim3 grid(blocks), block(kThreads);
    if (dt == kBF16) {
        if (aligned) hipLaunchKernelGGL((k_stats_tree_sample<kBF16, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_stats_tree_sample<kBF16, false>), grid, block, 0, s, p);
    } else {
        if (aligned) hipLaunchKernelGGL((k_stats_tree_sample<kF32, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_stats_tree_sample<kF32, false>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_tree_round(const RoundParams& p, Dt dt, bool aligned, hipStream_t s) {
    const unsigned blocks = (unsigned)((long long)p.B * p.NCd);
    const dim3 grid(blocks), block(kThreads);
    if (dt == kBF16) {
        if (aligned) hipLaunchKernelGGL((k_tree_round<kBF16, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_tree_round<kBF16, false>), grid, block, 0, s, p);
    } else {
        if (aligned) hipLaunchKernelGGL((k_tree_round<kF32, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_tree_round<kF32, false>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_draw(const DrawParams& p, Dt dt, bool aligned, hipStream_t s) {
    const unsigned blocks = (unsigned)((long long)p.B * p.NCd);
    const dim3 grid(blocks), block(kThreads);
    if (dt == kBF16) {
        if (aligned) hipLaunchKernelGGL((k_draw<kBF16>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_draw_unaligned<kBF16>), grid, block, 0, s, p);
    } else {
        if (aligned) hipLaunchKernelGGL((k_draw<kF32>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_draw_unaligned<kF32>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_mtp(const MtpParams& p, bool aligned, hipStream_t s) {
    const long long work_tok = p.B;
    const long long copy_blocks = (p.hsrc && p.hdst && p.hsrc != p.hdst)
                                      ? (p.hidden_elems / 8 + (long long)kThreads * SV_COPY_VECS - 1) /
                                            ((long long)kThreads * SV_COPY_VECS)
                                      : 0;
    const long long tok_blocks = (work_tok + kThreads - 1) / kThreads;
    long long blocks = copy_blocks > tok_blocks ? copy_blocks : tok_blocks;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (aligned) hipLaunchKernelGGL((k_mtp<true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_mtp<false>), grid, block, 0, s, p);
    return hipGetLastError();
}

hipError_t launch_clear(void* ws, size_t bytes, hipStream_t s) {
    const long long nvec = (long long)(bytes / 16);
    const int ntail = (int)(bytes % 16);
    long long blocks = (nvec + kThreads - 1) / kThreads;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_clear, dim3((unsigned)blocks), dim3(kThreads), 0, s, (uint4*)ws, nvec,
                       (uint8_t*)ws + nvec * 16, ntail);
    return hipGetLastError();
}

hipError_t launch_softmax_debug(const void* logits, Dt dt, const float* temp, int rows, int V, float* out,
                                bool aligned, hipStream_t s) {
    const dim3 grid((unsigned)rows), block(kThreads);
    if (dt == kBF16) {
        if (aligned) hipLaunchKernelGGL((k_softmax_debug<kBF16, true>), grid, block, 0, s, logits, temp, V, out);
        else hipLaunchKernelGGL((k_softmax_debug<kBF16, false>), grid, block, 0, s, logits, temp, V, out);
    } else {
        if (aligned) hipLaunchKernelGGL((k_softmax_debug<kF32, true>), grid, block, 0, s, logits, temp, V, out);
        else hipLaunchKernelGGL((k_softmax_debug<kF32, false>), grid, block, 0, s, logits, temp, V, out);
    }
    return hipGetLastError();
}

}  // namespace sv
