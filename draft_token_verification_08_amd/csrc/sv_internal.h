// sv_internal.h -- layouts and launch parameters shared by the kernels
// (sv_kernels.hip) and the host ABI layer (sv_api.cpp) of libspecverify.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "specverify.h"

namespace sv {

// Compile-time tuning knobs (defaults are the measured best on MI355X).
#ifndef SV_THREADS
#define SV_THREADS 256
#endif
#ifndef SV_TARGET_WORKGROUPS
#define SV_TARGET_WORKGROUPS 1024
#endif

constexpr int kThreads = SV_THREADS; // workgroup size of every kernel (wave64s)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxDraft = 64;        // n <= kMaxDraft
constexpr int kMaxSlots = 2 * kMaxDraft + 1;
#ifndef SV_DRAW_TILES
#define SV_DRAW_TILES 8
#endif
constexpr int kDrawTiles = SV_DRAW_TILES;  // draw pass: tiles (kThreads * elements per 16-byte vector) per chunk
constexpr int kMaxTiles = 1024;      // tiles per row (4 per thread in the draw selections)
constexpr int kTargetWorkgroups = SV_TARGET_WORKGROUPS;  // stats pass: workgroups over the target rows
constexpr int kMaxPartials = 2048;       // (2n+1) * chunks per row, staged in LDS by the decision
constexpr int kDrawSums = 6;         // per-tile sums a residual draw chunk hands over (far form: the first 4)

enum Dt : int { kF32 = 0, kBF16 = 1 };
enum Mode : int { kSample = 0, kGreedy = 1 };

// kinds of the final draw of a sequence: a bonus draw from target row L's tile
// partials, a residual draw max(0, p_k - lam q_k) from row pair k, or a draw
// from the whole of target row k alone (the bonus token at a tree's leaf).
// kDrawResidualNear is a residual draw whose mass may be small (below the near
// form's threshold): its chunks hand over the near form's tile sums instead of
// the far form's.
enum DrawKind : int { kDrawNone = 0, kDrawBonus = 1, kDrawResidual = 2, kDrawTarget = 3, kDrawResidualNear = 4 };
__host__ __device__ inline bool is_residual_draw(int kind) { return kind == kDrawResidual || kind == kDrawResidualNear; }

// One 64-bit slot per (sequence, row slot, vocab chunk), exchanged atomically:
//   sampling rows: low word chunk max m_c, high word sum over the chunk of 2^((z - m_c) c)
//   greedy rows:   chunk slot 0 holds the row's argmax key (atomic max over chunks)
struct Partial {
    float a;
    float b;
};

// Per sequence, written by the decision and read by the draw pass.  A zero
// descriptor is kDrawNone.
struct DrawDesc {
    int kind;       // DrawKind
    int k;          // row index of the draw (target row k, and draft row k if residual)
    int slot;       // output slot of the drawn token (emitted[b][slot])
    float c;        // log2(e) / T as used for every exponent of this sequence
    float m_t;      // max of target row k
    float m_d;      // max of draft row k (residual only)
    float lq;       // log2(S_t / S_d), S = sum 2^((z - m) c) of target / draft row k (residual only)
    float u;        // the (sanitised) final uniform u[b][n]
    double mu;      // residual draws: the weights are max(0, p - lam q) with lam = 1 + mu (mu = 0
                    // after one rejection; tree walks: more), mu itself when at least 2^-1000,
                    // else log2(mu) (< -1000)
    double lkap;    // skap != 0: log2 |kappa|, kappa = S_d / S_t - lam (-inf: kappa = 0)
    int skap;       // the sign of kappa (+1 or -1) when a tree walk carries it (after two or
                    // more rejections at a node); 0: kappa = S_d / S_t - 1, formed by the draw
    int pad_;
};
static_assert(sizeof(DrawDesc) == 56, "the workspace layout sizes DrawDesc at 56 bytes");

// A sampling tree walk (per sequence), kept in the workspace between the
// statistics pass, the rounds and the draw pass.
enum WalkStatus : int { kWalkIdle = 0, kWalkPending = 1 };
struct TreeWalk {
    int status;     // WalkStatus: pending = the walk needs M at lam for node u
    int u;          // current node
    int next;       // the next child to test is the first node j + 1 with j >= next below u
    int depth;      // nodes on the kept path so far
    double zb;      // a lower bound of sum max(0, p_u - lam_k q_u) (< 0: no child rejected yet)
    double lmu;     // log2(lam_k - 1) once a child is rejected (-inf: lam_k = 1)
    double lkap;    // skap != 0: log2 |kappa_k|, kappa_k = S_d / S_t - lam_k at node u (-inf: 0)
    int skap;       // the sign of kappa_k once two children at u are rejected; 0: not carried
    uint32_t flags;
    float c;        // log2(e) / T
    int path[kMaxDraft];
};

// Per-sequence rows of a sampling tree walk: the statistics of target rows
// 0..n and draft rows 0..n-1, and each node's gathered logits (node j + 1:
// target and draft logit of x_j in its parent's rows).  Byte offsets inside a
// sequence's block of tree_rows_stride(n) bytes.
struct TreeRowsLayout {
    int mt, St, md, Sd, gt, gd, stride;
};
__host__ __device__ inline TreeRowsLayout tree_rows_layout(int n) {
    auto up8 = [](int x) { return (x + 7) / 8 * 8; };
    TreeRowsLayout l;
    l.mt = 0;
    l.St = up8(4 * (n + 1));
    l.md = l.St + 8 * (n + 1);
    l.Sd = up8(l.md + 4 * n);
    l.gt = l.Sd + 8 * n;
    l.gd = l.gt + 4 * n;
    l.stride = (l.gd + 4 * n + 15) / 16 * 16;
    return l;
}

// Workspace layout (byte offsets from the workspace base; every region 256-aligned).
struct Layout {
    int NC;          // vocab chunks per row in the stats pass
    int CH;          // elements per stats chunk (multiple of the vector tile)
    int NT;          // tiles per row (kThreads * elements per 16-byte vector each)
    int NCd;         // chunks of kDrawTiles tiles per row in the draw pass
    size_t off_part;     // Partial [B][2n+1][NC]
    size_t off_cnt;      // uint32 [B]   stats-pass arrival counters
    size_t off_cnt_draw; // uint32 [B]   draw-pass arrival counters
    size_t off_desc;     // DrawDesc [B]
    size_t off_tiles;    // uint64 [B][NT] tile partials (m_t, s_t) of target row L (sampling)
    size_t off_dsum;     // float [B][kDrawSums][NT] per-tile sums of the residual draw (draw pass)
    size_t off_walk;     // TreeWalk [B] (sampling tree walks)
    size_t off_trows;    // [B][tree_rows_layout(n).stride] bytes (sampling tree walks)
    size_t off_acc;      // int32 [B] accepted lengths of sv_sample_rows (always 0)
    size_t bytes;
};

// MTP bookkeeping fused into the verify kernels: the token shift/insert and the
// hidden-state carry of one decode step.  tokens == nullptr disables it; hsrc ==
// nullptr (or nvec == 0) skips the copy.
struct MtpFuse {
    int32_t* tokens;          // [B][n+1] or nullptr
    const void* hsrc;         // nvec 16-byte vectors (bf16 hidden states), or nullptr
    void* hdst;
    long long nvec;
};

struct StatsParams {
    const void* target;       // [B][n+1][V]
    const void* draft;        // [B][n][V] or nullptr
    const int32_t* tokens;    // [B][n]
    const int32_t* lens;      // [B]
    const float* temp;        // [B] (sample mode)
    const float* unif;        // [B][n+1] (sample mode)
    int B, n, V, NC, CH, S;   // S = row slots per sequence (2n+1 sample, n+1 greedy)
    int NT;                   // tiles per row
    unsigned long long* tiles;  // [B][NT] tile partials (m_t, s_t) of target row L
    int R;                    // target rows per sequence in memory (n + 1, or R of sv_sample_rows)
    const int32_t* row_index; // [B] or nullptr: target row 0 of sequence b is row_index[b] (clamped)
    int32_t* acc;             // [B]
    int32_t* emitted;         // [B][n+1]
    float* row_lse;           // [B][2n+1] or nullptr
    uint32_t* flags;          // [1] or nullptr
    Partial* part;
    uint32_t* cnt;
    DrawDesc* desc;
    MtpFuse mtp;              // zero: not fused
    const float* dstats;      // [B][n][2] {max, sum 2^((z - max) c)} of the draft rows, from the
                              // draft's own sampling step, or nullptr (draft rows are then streamed)
    float* out_stats;         // [B][2] or nullptr: the same statistics of the row of target slot 0
    int draw_in_stats;        // 1 (n == 0 only): the decision makes the bonus draw itself and no
                              // draw pass runs; row 0's tile partials are then exchanged atomically
    const int32_t* parents;   // [B][n] tree verification: node j + 1 hangs below node parents[j]
    int32_t* path;            // [B][n] or nullptr: the kept path's node indices (tree verification)
    TreeWalk* walk;           // [B] sampling tree walks
    char* trows;              // [B][stride] sampling tree walks' rows
    int can_pend;             // a sampling tree walk may stop to wait for a round (rounds follow)
};

// One round of the sampling tree walks: the residual mass of every pending
// walk's row pair, then the walk goes on.
struct RoundParams {
    const void* target;       // [B][n+1][V]
    const void* draft;        // [B][n][V]
    const int32_t* tokens;    // [B][n]
    const int32_t* parents;   // [B][n]
    const int32_t* lens;      // [B]
    const float* unif;        // [B][n+1]
    int B, n, V, NT, NCd;
    TreeWalk* walk;
    char* trows;
    int can_pend;             // not the last round
    float* dsum;              // [B][kDrawSums][NT]
    uint32_t* cnt;            // [B]
    DrawDesc* desc;           // [B]
    int32_t* acc;
    int32_t* emitted;
    int32_t* path;            // or nullptr
    uint32_t* flags;          // or nullptr
};

struct DrawParams {
    const void* target;
    const void* draft;
    int B, n, V, NT, NCd;
    int R;
    const int32_t* row_index;
    unsigned long long* tiles;
    int32_t* emitted;
    uint32_t* flags;
    DrawDesc* desc;
    float* dsum;              // [B][kDrawSums][NT]
    uint32_t* cnt;
    int32_t* mtp_tokens;      // [B][n+1] or nullptr: the drawn token is also written to slot k
};

struct MtpParams {
    int32_t* tokens;          // [B][n+1]
    const void* hsrc;         // [B][n+1][H] bf16 or nullptr
    void* hdst;
    long long hidden_elems;   // B*(n+1)*H
    const int32_t* acc;
    const int32_t* emitted;
    int B, n;
};

// The target's logit projection (lm_head) on the bf16 matrix cores:
// logits[m][v] = sum_k hidden[m][k] * weight[v][k], accumulated in binary32.
// With `keys` set the logits stay in registers: each workgroup reduces its
// tile to a per-row (max, lowest index) and merges it into keys[m] by atomic
// max; with `logits` set they are stored (parity/debug).
struct LmParams {
    const void* hidden;        // [M][H] bf16, 16-byte aligned, H a multiple of kLmBK
    const void* weight;        // [V][H] bf16, 16-byte aligned
    int M, H, V;
    float* logits;             // [M][V] or nullptr
    unsigned long long* keys;  // [M] or nullptr
    const int32_t* lens;       // [B] with keys: row m = b*(n+1) + r is needed iff r <= clamp(lens[b], 0, n)
    int n;
    void* hidden_dst;          // nullptr or [M][H]: the hidden-state carry of the MTP step
};
constexpr int kLmBK = 64;      // K elements per pipeline stage of the projection

// Host layer (sv_api.cpp): the body of spec_verify_sample_ex() on a given
// workspace, and the SV_EHIP status for a HIP error (its text recorded for
// sv_last_hip_error()).
sv_status_t sample_ex(const void* target_logits, const void* draft_logits, sv_dtype_t dt, const int32_t* draft_tokens,
                      const int32_t* draft_lens, const float* temperature, const float* uniforms,
                      const float* draft_stats, int B, int n, int V, int32_t* accepted_len, int32_t* emitted,
                      float* row_lse, uint32_t* err_flags, int32_t* tokens, const void* hidden_src, void* hidden_dst,
                      int H, void* workspace, size_t workspace_bytes, void* stream);
sv_status_t hip_status(hipError_t e);

// launches (sv_kernels.hip, sv_lmhead.hip); return the hipGetLastError() after the launch
hipError_t launch_stats(const StatsParams& p, Dt dt, Mode mode, bool aligned, hipStream_t s);
hipError_t launch_tree(const StatsParams& p, Dt dt, bool aligned, hipStream_t s);
hipError_t launch_tree_sample(const StatsParams& p, Dt dt, bool aligned, hipStream_t s);
hipError_t launch_tree_round(const RoundParams& p, Dt dt, bool aligned, hipStream_t s);
hipError_t launch_draw(const DrawParams& p, Dt dt, bool aligned, hipStream_t s);
hipError_t launch_mtp(const MtpParams& p, bool aligned, hipStream_t s);
hipError_t launch_clear(void* ws, size_t bytes, hipStream_t s);
hipError_t launch_lmhead(const LmParams& p, hipStream_t s);
hipError_t launch_decide_greedy(const StatsParams& p, hipStream_t s);
hipError_t launch_residual_debug(const void* target, const void* draft, Dt dt, const float* temp, int rows, int V,
                                 int NT, float* w_out, double* tile_out, float* info_out, bool aligned,
                                 hipStream_t s);
hipError_t launch_softmax_debug(const void* logits, Dt dt, const float* temp, int rows, int V,
                                float* out, bool aligned, hipStream_t s);

}  // namespace sv
