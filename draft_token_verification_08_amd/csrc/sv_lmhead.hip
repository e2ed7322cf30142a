// sv_lmhead.hip -- the target's logit projection (its lm_head) on the gfx950
// bf16 matrix cores, fused with the greedy verify's row reduction.
//
// "Accelerating Sonar through speculation": the model runs to produce logits
// from which the next token is sampled (Inference with speculative decoding
// section, first paragraph), through a logit projection that the MTP head
// reuses and that is about 2 GB for a 70B Llama (MTP section, the paragraph on
// the head's normalisation layers).  A greedy verify needs only each row's
// (max, lowest index), so the [B, n+1, V] logits never have to reach memory:
// every workgroup reduces its tile of logits in registers and merges one
// 64-bit key per row by atomic max; the per-sequence decision then runs on the
// keys (k_decide_greedy).
//
// The product is logits[m][v] = sum_k hidden[m][k] * weight[v][k], hidden
// [M][H] and weight [V][H] both K-contiguous bf16, accumulated in binary32 by
// the bf16 matrix cores (lane layouts of both instruction shapes checked on
// MI355X; see Mfma below).  Both operands of a lane are 16 contiguous bytes of
// a K-contiguous row: one ds_read_b128 each.
//
// Workgroup tile BM x BN = 256 x 256 by default: 8 waves (2 along the rows, 4
// along the vocabulary), each a 128 x 64 block held in 8 x 4 accumulators of
// 16 x 16 (v_mfma_f32_16x16x32_bf16, 128 registers), so a workgroup per CU
// runs two waves per SIMD.  K runs in stages of 64.  A stage's A and B rows
// are loaded to registers with 16-byte loads (8 lanes per 128-byte row
// segment) and written to LDS with a 32-byte pad per row (rows 160 bytes
// apart, so the lanes of a fragment read hit distinct banks; the two stage
// buffers then fill the 160 KB of LDS exactly).  The two buffers alternate:
// while the waves run the MFMAs of stage kt from one, stage kt+1 is stored to
// the other and stage kt+2 loaded, with one barrier per stage.  Tile
// shape, matrix-core shape, buffering, scheduling strategy and tile order are
// compile-time knobs; the defaults are the fastest measured on MI355X.
#include <cfloat>
#include <climits>
#include <cmath>

#include "sv_internal.h"
#include "sv_device.h"

#ifndef SV_LM_WM
#define SV_LM_WM 2  // waves along the hidden rows
#endif
#ifndef SV_LM_WN
#define SV_LM_WN 4  // waves along the vocabulary
#endif
#ifndef SV_LM_WTM
#define SV_LM_WTM 4  // 32-row units per wave
#endif
#ifndef SV_LM_WTN
#define SV_LM_WTN 2  // 32-column units per wave
#endif
#ifndef SV_LM_WPE
#define SV_LM_WPE 2  // waves per SIMD the register budget is sized for
#endif
#ifndef SV_LM_MFMA
#define SV_LM_MFMA 16  // matrix-core block edge: 32 (32x32x16) or 16 (16x16x32)
#endif
#ifndef SV_LM_IGLP
#define SV_LM_IGLP 1  // instruction-group scheduling strategy for the MFMA loop (-1: none)
#endif
#ifndef SV_LM_PAD
#define SV_LM_PAD 32  // LDS row pad in bytes (a multiple of 16)
#endif
#ifndef SV_LM_XCD
#define SV_LM_XCD 1  // XCD-aware tile order
#endif
#ifndef SV_LM_LDSBUF
#define SV_LM_LDSBUF 2  // LDS stages: 1 (two barriers per stage) or 2 (double buffer, one barrier)
#endif

namespace sv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));  // one 16-byte load (a native vector)

typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS bytes per tile row: one stage of K plus a pad.  The pad decides the
// bank pattern of the fragment reads (rows (lane % 16), 16-byte chunk lane / 16
// for the 16 x 16 blocks): measured on MI355X, 144-byte rows give 2-way bank
// conflicts for that pattern and 160-byte rows none.
constexpr int kPitch = kLmBK * 2 + SV_LM_PAD;
__device__ __forceinline__ int lds_off(int r, int c) { return r * kPitch + (c << 4); }

// The two bf16 matrix-core shapes.  Both take 8 bf16 per lane per operand
// (16 contiguous bytes of a K-contiguous row): lane l holds row (or column)
// l % S at k = (l / S) * 8 + e.  Accumulator register r of lane l is column
// l % S and row row_of(l, r).
template <int S_>
struct Mfma;
template <>
struct Mfma<32> {  // v_mfma_f32_32x32x16_bf16: 32 x 32 block, 16 k per instruction
    static constexpr int S = 32, K = 16, NR = 16;
    using acc_t = f32x16;
    __device__ static acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static int row_of(int lane, int r) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }
    // argmax over the lanes that share a row set (the 32 lanes of a half wave)
    __device__ static ArgMax reduce(ArgMax a) { return half_wave_argmax(a); }
};
template <>
struct Mfma<16> {  // v_mfma_f32_16x16x32_bf16: 16 x 16 block, 32 k per instruction
    static constexpr int S = 16, K = 32, NR = 4;
    using acc_t = f32x4;
    __device__ static acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static int row_of(int lane, int r) { return (lane >> 4) * 4 + r; }
    // argmax over the 16 lanes of a DPP row
    __device__ static ArgMax reduce(ArgMax a) {
        a = better(a, dpp_am<kDppXor1>(a));
        a = better(a, dpp_am<kDppXor2>(a));
        a = better(a, dpp_am<kDppHalfMirror>(a));
        a = better(a, dpp_am<kDppMirror>(a));
        return a;
    }
};
using MF = Mfma<SV_LM_MFMA>;

template <int WM_, int WN_>
struct Tile {
    static constexpr int WM = WM_, WN = WN_;
    static constexpr int TM = SV_LM_WTM, TN = SV_LM_WTN;  // 32 x 32 units per wave
    static constexpr int QM = 32 * TM / MF::S, QN = 32 * TN / MF::S;  // accumulator blocks per wave
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int BM = 32 * TM * WM;        // hidden rows per workgroup
    static constexpr int BN = 32 * TN * WN;        // vocabulary entries per workgroup
    static constexpr int kRowStep = kThreads / 8;  // rows one pass of 16-byte loads covers
    static constexpr int kA = BM / kRowStep;       // 16-byte loads per thread per stage (hidden)
    static constexpr int kB = BN / kRowStep;       // (weight)
    static constexpr int kLds = (BM + BN) * kPitch;  // one stage
    static_assert(BM % kRowStep == 0 && BN % kRowStep == 0, "tile rows per load pass");
};

// Tile number of this workgroup.  Workgroups are dealt to the 8 XCDs in turn
// (XCD = workgroup id mod 8).  XCD x takes the contiguous tile numbers
// [start_x, start_x + count_x), and tile numbers run over the row tiles first,
// so the row tiles that share a weight tile run on one XCD at about the same
// time and read that weight tile through its L2 once.
__device__ __forceinline__ int tile_of_workgroup() {
    const int G = gridDim.x, bid = blockIdx.x;
    const int q = G >> 3, rem = G & 7, x = bid & 7;
    return SV_LM_XCD ? x * q + min(x, rem) + (bid >> 3) : bid;
}

// The MTP hidden-state carry: every workgroup copies an equal share of the
// [M][H] hidden states (16-byte vectors) after its tile.
__device__ __forceinline__ void hidden_copy_share(const LmParams& p) {
    if (p.hidden_dst == nullptr) return;
    const long long nvec = (long long)p.M * (p.H / 8);
    const long long share = (nvec + gridDim.x - 1) / gridDim.x;
    const long long v0 = (long long)blockIdx.x * share;
    const long long v1 = min(nvec, v0 + share);
    const v4u* src = static_cast<const v4u*>(p.hidden);
    v4u* dst = static_cast<v4u*>(p.hidden_dst);
    for (long long v = v0 + threadIdx.x; v < v1; v += blockDim.x) dst[v] = src[v];
}

// After the main loop: store the tile's logits (debug) or reduce each row to
// (max, lowest index) over this wave's columns, then over the WN waves of the
// row tile, and merge it into keys[m] across tiles.  `scratch` is LDS the main
// loop no longer reads (at least WN * BM * 8 bytes).
template <class T, bool KEYS>
__device__ __forceinline__ void lmhead_epilogue(const LmParams& p, const typename MF::acc_t (&acc)[T::QM][T::QN],
                                                unsigned char* scratch, int m0, int n0) {
    constexpr int TM = T::TM, TN = T::TN, QM = T::QM, QN = T::QN, WN = T::WN, S = MF::S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % T::WM, wn = wave / T::WM;
    if constexpr (!KEYS) {
#pragma unroll
        for (int bm = 0; bm < QM; ++bm)
#pragma unroll
            for (int bn = 0; bn < QN; ++bn)
#pragma unroll
                for (int r = 0; r < MF::NR; ++r) {
                    const int i = m0 + wm * 32 * TM + bm * S + MF::row_of(lane, r);
                    const int j = n0 + wn * 32 * TN + bn * S + (lane % S);
                    if (i < p.M && j < p.V) p.logits[(size_t)i * p.V + j] = acc[bm][bn][r];
                }
    } else {
        unsigned long long* s_key = reinterpret_cast<unsigned long long*>(scratch);  // [WN][BM]
#pragma unroll
        for (int bm = 0; bm < QM; ++bm)
#pragma unroll
            for (int r = 0; r < MF::NR; ++r) {
                ArgMax a{-INFINITY, INT_MAX};
#pragma unroll
                for (int bn = 0; bn < QN; ++bn) {
                    const int j = n0 + wn * 32 * TN + bn * S + (lane % S);
                    if (j < p.V) a = better(a, ArgMax{acc[bm][bn][r], j});
                }
                a = MF::reduce(a);
                if ((lane % S) == 0) s_key[wn * T::BM + wm * 32 * TM + bm * S + MF::row_of(lane, r)] = argmax_key(a);
            }
        __syncthreads();
        for (int i = tid; i < T::BM; i += T::kThreads) {
            const int m = m0 + i;
            if (m >= p.M) continue;
            const int b = m / (p.n + 1), r = m - b * (p.n + 1);
            const int L = min(max(p.lens[b], 0), p.n);
            if (r > L) continue;  // rows past the draft length take no part in the decision
            unsigned long long k = s_key[i];
#pragma unroll
            for (int w = 1; w < WN; ++w) k = max(k, s_key[w * T::BM + i]);
            max64(p.keys + m, k);
        }
        hidden_copy_share(p);
    }
}

template <int WM, int WN, bool KEYS>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(SV_LM_WPE, SV_LM_WPE)))
void k_lmhead(LmParams p, int tiles_m) {
    using T = Tile<WM, WN>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[T::kLds * SV_LM_LDSBUF];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;

    const int tile = tile_of_workgroup();
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int m0 = tm * T::BM, n0 = tn * T::BN;

    // this thread's 16-byte loads: column lcol of rows lrow + i * kRowStep.
    // Rows past M (or V) in the last tiles load the last row again: their
    // products land in accumulator rows (columns) that are never stored or
    // reduced, so no zero fill is needed and every load stays in bounds.
    const int lrow = tid >> 3, lcol = tid & 7;
    const unsigned vrow = (unsigned)(p.H / 8);  // 16-byte vectors per row
    const v4u* const A = static_cast<const v4u*>(p.hidden);
    const v4u* const W = static_cast<const v4u*>(p.weight);
    unsigned aoff[T::kA], boff[T::kB];
#pragma unroll
    for (int i = 0; i < T::kA; ++i)
        aoff[i] = (unsigned)min(m0 + lrow + i * T::kRowStep, p.M - 1) * vrow + lcol;
#pragma unroll
    for (int i = 0; i < T::kB; ++i)
        boff[i] = (unsigned)min(n0 + lrow + i * T::kRowStep, p.V - 1) * vrow + lcol;

    v4u ra[T::kA], rb[T::kB];
#pragma unroll
    for (int i = 0; i < T::kA; ++i) ra[i] = A[aoff[i]];
#pragma unroll
    for (int i = 0; i < T::kB; ++i) rb[i] = W[boff[i]];

    constexpr int TM = T::TM, TN = T::TN, QM = T::QM, QN = T::QN, S = MF::S;
    typename MF::acc_t acc[QM][QN];
#pragma unroll
    for (int bm = 0; bm < QM; ++bm)
#pragma unroll
        for (int bn = 0; bn < QN; ++bn)
#pragma unroll
            for (int r = 0; r < MF::NR; ++r) acc[bm][bn][r] = 0.f;

    const int KT = p.H / kLmBK;
    auto store_stage = [&](unsigned char* buf) {
#pragma unroll
        for (int i = 0; i < T::kA; ++i)
            *reinterpret_cast<v4u*>(buf + lds_off(lrow + i * T::kRowStep, lcol)) = ra[i];
#pragma unroll
        for (int i = 0; i < T::kB; ++i)
            *reinterpret_cast<v4u*>(buf + lds_off(T::BM + lrow + i * T::kRowStep, lcol)) = rb[i];
    };
    auto load_stage = [&](int kt) {
        const unsigned o = (unsigned)kt * (kLmBK / 8);
#pragma unroll
        for (int i = 0; i < T::kA; ++i) ra[i] = A[aoff[i] + o];
#pragma unroll
        for (int i = 0; i < T::kB; ++i) rb[i] = W[boff[i] + o];
    };
    auto load_frags = [&](const unsigned char* buf, int s, bf16x8* fa, bf16x8* fb) {
        const int kc = s * (MF::K / 8) + lane / S;  // 16-byte chunk of this lane's 8 k values
#pragma unroll
        for (int bm = 0; bm < QM; ++bm)
            fa[bm] = *reinterpret_cast<const bf16x8*>(buf + lds_off(wm * 32 * TM + bm * S + (lane % S), kc));
#pragma unroll
        for (int bn = 0; bn < QN; ++bn)
            fb[bn] = *reinterpret_cast<const bf16x8*>(buf + lds_off(T::BM + wn * 32 * TN + bn * S + (lane % S), kc));
    };
    auto compute_stage = [&](const unsigned char* buf) {
#if SV_LM_IGLP >= 0
        __builtin_amdgcn_iglp_opt(SV_LM_IGLP);  // the compiler's MFMA / LDS-read interleaving strategy
#endif
#pragma unroll
        for (int s = 0; s < kLmBK / MF::K; ++s) {
            bf16x8 fa[QM], fb[QN];
            load_frags(buf, s, fa, fb);
#pragma unroll
            for (int bm = 0; bm < QM; ++bm)
#pragma unroll
                for (int bn = 0; bn < QN; ++bn) acc[bm][bn] = MF::mma(fa[bm], fb[bn], acc[bm][bn]);
        }
    };
#if SV_LM_LDSBUF == 1
    // one LDS stage: store, barrier, issue the next stage's loads, compute, barrier
    for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();  // every wave has read the previous stage
        store_stage(lds);
        __syncthreads();
        if (kt + 1 < KT) load_stage(kt + 1);
        compute_stage(lds);
    }
#else
    // two LDS stages: while the waves compute stage kt from one buffer, stage
    // kt+1 (already in registers) is stored to the other and stage kt+2 loaded;
    // one barrier per stage
    store_stage(lds);
    if (KT > 1) load_stage(1);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) {
            store_stage(lds + ((kt + 1) & 1) * T::kLds);
            if (kt + 2 < KT) load_stage(kt + 2);
        }
        compute_stage(lds + (kt & 1) * T::kLds);
        __syncthreads();
    }
#endif

    if constexpr (KEYS) __syncthreads();  // the last stage's fragment reads are done: reuse the LDS
    lmhead_epilogue<T, KEYS>(p, acc, lds, m0, n0);
}

template <int WM, int WN, bool KEYS>
hipError_t launch_tiles(const LmParams& p, hipStream_t s) {
    using T = Tile<WM, WN>;
    const long long tm = (p.M + T::BM - 1) / T::BM;
    const long long tn = ((long long)p.V + T::BN - 1) / T::BN;
    const long long G = tm * tn;
    if (G == 0) return hipSuccess;
    if (G > INT_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_lmhead<WM, WN, KEYS>), dim3((unsigned)G), dim3(T::kThreads), 0, s, p, (int)tm);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead(const LmParams& p, hipStream_t s) {
    if (p.H % kLmBK != 0 || p.H < kLmBK) return hipErrorInvalidValue;
    return p.keys ? launch_tiles<SV_LM_WM, SV_LM_WN, true>(p, s) : launch_tiles<SV_LM_WM, SV_LM_WN, false>(p, s);
}

}  // namespace sv
