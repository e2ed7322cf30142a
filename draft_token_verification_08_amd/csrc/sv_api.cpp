// sv_api.cpp -- the C ABI of libspecverify: argument checks, workspace layout and
// launch configuration.  Every check here uses host-visible values only; nothing
// reads device memory and nothing synchronises.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "sv_internal.h"

namespace {

thread_local char g_hip_error[256] = "";

sv_status_t hip_fail(hipError_t e) {
    std::snprintf(g_hip_error, sizeof g_hip_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return SV_EHIP;
}

size_t elem_bytes(sv_dtype_t dt) { return dt == SV_BF16 ? 2 : 4; }
int vec_elems(sv_dtype_t dt) { return dt == SV_BF16 ? 8 : 4; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

bool aligned_to(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_sizes(int B, int n, int V) {
    return B >= 0 && n >= 0 && n <= sv::kMaxDraft && V >= 1;
}

// Chunking of rows over workgroups.  Depends on (B, n, V, dt) only, so the
// sample and greedy entry points agree with sv_workspace_bytes().
//   stats pass: enough chunks that ~kTargetWorkgroups workgroups cover the
//     B*(n+1) target rows; chunk length a multiple of one vector per thread.
//   draw pass: tiles of kThreads * (elements per 16-byte vector), kDrawTiles per chunk.
bool make_layout(int B, int n, int V, sv_dtype_t dt, sv::Layout* L) {
    const long long tile = (long long)sv::kThreads * vec_elems(dt);
    const long long rows_t = (long long)B * (n + 1);
    long long nc = rows_t > 0 ? ceil_div(sv::kTargetWorkgroups, rows_t) : 1;
    const long long nc_max = ceil_div(V, tile);
    if (nc > nc_max) nc = nc_max;
    const long long nc_lds = sv::kMaxPartials / (2 * n + 1);  // partials staged in LDS by the decision
    if (nc > nc_lds) nc = nc_lds;
    if (nc < 1) nc = 1;
    long long ch = ceil_div(ceil_div(V, nc), tile) * tile;
    nc = ceil_div(V, ch);
    const long long nt = ceil_div(V, tile);
    const long long ncd = ceil_div(nt, sv::kDrawTiles);
    if (nt > sv::kMaxTiles) return false;
    L->NC = (int)nc;
    L->CH = (int)ch;
    L->NT = (int)nt;
    L->NCd = (int)ncd;
    const size_t slots = (size_t)(2 * n + 1);
    size_t off = 0;
    L->off_part = off;
    off = align_up(off + (size_t)B * slots * nc * sizeof(sv::Partial), 256);
    L->off_cnt = off;
    off = align_up(off + (size_t)B * sizeof(uint32_t), 256);
    L->off_cnt_draw = off;
    off = align_up(off + (size_t)B * sizeof(uint32_t), 256);
    L->off_desc = off;
    off = align_up(off + (size_t)B * sizeof(sv::DrawDesc), 256);
    L->off_tiles = off;
    off = align_up(off + (size_t)B * nt * sizeof(unsigned long long), 256);
    L->off_dsum = off;
    off = align_up(off + (size_t)B * sv::kDrawSums * nt * sizeof(float), 256);
    L->off_walk = off;
    off = align_up(off + (size_t)B * sizeof(sv::TreeWalk), 256);
    L->off_trows = off;
    off = align_up(off + (size_t)B * sv::tree_rows_layout(n).stride, 256);
    L->off_acc = off;
    off = align_up(off + (size_t)B * sizeof(int32_t), 256);
    L->bytes = off < 256 ? 256 : off;
    return true;
}

#ifndef SV_DRAW_IN_STATS
#define SV_DRAW_IN_STATS 1  // calls with no drafts make their draws in the stats pass's decision
#endif

template <class T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// grid sizes stay within one 32-bit dimension of 256-thread workgroups
bool grid_ok(long long blocks) { return blocks >= 0 && blocks * sv::kThreads <= 0xFFFFFFFFll; }

bool rows_aligned(const void* base, int V, sv_dtype_t dt) {
    return aligned_to(base, 16) && ((size_t)V * elem_bytes(dt)) % 16 == 0;
}

// Byte range of a caller buffer, for the aliasing checks of the fused calls.
struct Span {
    const void* p;
    size_t bytes;
};

bool overlap(Span a, Span b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool overlaps_any(Span a, const Span* others, int k) {
    for (int i = 0; i < k; ++i)
        if (overlap(a, others[i])) return true;
    return false;
}

// Hidden-state element count B * (n+1) * H, or -1 when it does not fit the
// byte range of the address space.
long long hidden_elems(int B, int n, int H) {
    const long long rows = (long long)B * (n + 1);
    if (H <= 0 || rows == 0) return 0;
    if (rows > (1ll << 62) / 2 / H) return -1;
    return rows * H;
}

// The MTP arguments of a fused verify + MTP call.
struct MtpArgs {
    int32_t* tokens;
    const void* hsrc;
    void* hdst;
    int H;
};

// Checks shared by mtp_shift_insert() and the fused calls; *elems receives the
// hidden element count (0 when there is nothing to copy).
sv_status_t check_mtp(const MtpArgs& m, int B, int n, long long* elems) {
    if (m.H < 0) return SV_EINVAL;
    if (!m.tokens) return SV_EINVAL;
    if ((m.hsrc == nullptr) != (m.hdst == nullptr)) return SV_EINVAL;
    if (m.hsrc && m.H < 1) return SV_EINVAL;
    if (!aligned_to(m.tokens, 4) || !aligned_to(m.hsrc, 2) || !aligned_to(m.hdst, 2)) return SV_EALIGN;
    const long long e = m.hsrc ? hidden_elems(B, n, m.H) : 0;
    if (e < 0) return SV_EINVAL;
    if (m.hsrc && m.hsrc != m.hdst && overlap(Span{m.hsrc, (size_t)e * 2}, Span{m.hdst, (size_t)e * 2}))
        return SV_EINVAL;  // partial overlap of the hidden buffers
    *elems = (m.hsrc == m.hdst) ? 0 : e;
    return SV_OK;
}

// Launch plan of the MTP part of a fused call: copy and token shift inside the
// verify kernels when the hidden buffers allow 16-byte vectors, else the
// separate MTP kernel after them.
struct MtpPlan {
    bool fused;
    sv::MtpFuse f;
    sv::MtpParams sep;
    bool sep_aligned;
};

MtpPlan plan_mtp(const MtpArgs& m, long long elems, const int32_t* accepted_len, const int32_t* emitted,
                 int B, int n) {
    MtpPlan pl{};
    const bool vec_ok = elems == 0 || (aligned_to(m.hsrc, 16) && aligned_to(m.hdst, 16) && elems % 8 == 0);
    pl.fused = vec_ok;
    if (pl.fused) {
        pl.f.tokens = m.tokens;
        pl.f.hsrc = elems > 0 ? m.hsrc : nullptr;
        pl.f.hdst = elems > 0 ? m.hdst : nullptr;
        pl.f.nvec = elems / 8;
    } else {
        pl.sep.tokens = m.tokens;
        pl.sep.hsrc = m.hsrc;
        pl.sep.hdst = m.hdst;
        pl.sep.hidden_elems = elems;
        pl.sep.acc = accepted_len;
        pl.sep.emitted = emitted;
        pl.sep.B = B;
        pl.sep.n = n;
        pl.sep_aligned = aligned_to(m.hsrc, 16) && aligned_to(m.hdst, 16);
    }
    return pl;
}

}  // namespace

extern "C" {

size_t sv_workspace_bytes(int B, int n, int V, sv_dtype_t dt) {
    if (!valid_sizes(B, n, V) || (dt != SV_F32 && dt != SV_BF16)) return 0;
    sv::Layout L;
    if (!make_layout(B, n, V, dt, &L)) return 0;
    return L.bytes;
}

sv_status_t sv_workspace_clear(void* workspace, size_t workspace_bytes, void* stream) {
    if (workspace_bytes == 0) return SV_OK;
    if (!workspace) return SV_EINVAL;
    if (!aligned_to(workspace, 16)) return SV_EALIGN;
    hipError_t e = sv::launch_clear(workspace, workspace_bytes, (hipStream_t)stream);
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

const char* sv_status_string(sv_status_t s) {
    switch (s) {
        case SV_OK: return "SV_OK: success";
        case SV_EINVAL: return "SV_EINVAL: invalid argument (NULL pointer or size out of range)";
        case SV_EALIGN: return "SV_EALIGN: pointer not aligned to its element type";
        case SV_EWORKSPACE: return "SV_EWORKSPACE: workspace missing or smaller than sv_workspace_bytes()";
        case SV_EHIP: return "SV_EHIP: HIP launch failed (see sv_last_hip_error())";
    }
    return "unknown status";
}

const char* sv_last_hip_error(void) { return g_hip_error; }

}  // extern "C"

namespace {

sv_status_t verify_sample(const void* target_logits, const void* draft_logits, sv_dtype_t dt,
                          const int32_t* draft_tokens, const int32_t* draft_lens, const float* temperature,
                          const float* uniforms, int B, int n, int V, int32_t* accepted_len, int32_t* emitted,
                          float* row_lse, uint32_t* err_flags, void* workspace, size_t workspace_bytes,
                          void* stream, const MtpArgs* mtp, const float* draft_stats) {
    if (!valid_sizes(B, n, V) || (dt != SV_F32 && dt != SV_BF16)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target_logits || !draft_lens || !temperature || !uniforms || !accepted_len || !emitted ||
        (n > 0 && !draft_tokens))
        return SV_EINVAL;
    const size_t es = elem_bytes(dt);
    if (!aligned_to(target_logits, es) || (draft_logits && !aligned_to(draft_logits, es)) ||
        !aligned_to(draft_tokens, 4) || !aligned_to(draft_lens, 4) || !aligned_to(temperature, 4) ||
        !aligned_to(uniforms, 4) || !aligned_to(accepted_len, 4) || !aligned_to(emitted, 4) ||
        !aligned_to(row_lse, 4) || !aligned_to(err_flags, 4) || !aligned_to(draft_stats, 4))
        return SV_EALIGN;
    if (draft_stats && !draft_logits) return SV_EINVAL;  // the gather and the residual need the rows
    sv::Layout L;
    if (!make_layout(B, n, V, dt, &L)) return SV_EINVAL;
    if (!workspace || workspace_bytes < L.bytes) return SV_EWORKSPACE;
    if (!aligned_to(workspace, 16)) return SV_EALIGN;
    const int S = 2 * n + 1;
    if (!grid_ok((long long)B * S * L.NC) || !grid_ok((long long)B * L.NCd)) return SV_EINVAL;

    MtpPlan pl{};
    if (mtp) {
        long long elems = 0;
        const sv_status_t ms = check_mtp(*mtp, B, n, &elems);
        if (ms != SV_OK) return ms;
        const size_t es_ = elem_bytes(dt);
        const Span tok{mtp->tokens, (size_t)B * (n + 1) * 4};
        const Span others[] = {{target_logits, (size_t)B * (n + 1) * V * es_},
                               {draft_logits, (size_t)B * n * V * es_},
                               {draft_tokens, (size_t)B * n * 4},
                               {draft_lens, (size_t)B * 4},
                               {temperature, (size_t)B * 4},
                               {uniforms, (size_t)B * (n + 1) * 4},
                               {accepted_len, (size_t)B * 4},
                               {emitted, (size_t)B * (n + 1) * 4},
                               {row_lse, row_lse ? (size_t)B * (2 * n + 1) * 4 : 0},
                               {draft_stats, draft_stats ? (size_t)B * n * 8 : 0},
                               {err_flags, err_flags ? 4u : 0u},
                               {workspace, workspace_bytes},
                               tok};
        constexpr int kOthers = sizeof(others) / sizeof(others[0]);
        if (overlaps_any(tok, others, kOthers - 1)) return SV_EINVAL;
        if (elems > 0 && overlaps_any(Span{mtp->hdst, (size_t)elems * 2}, others, kOthers)) return SV_EINVAL;
        pl = plan_mtp(*mtp, elems, accepted_len, emitted, B, n);
    }
    const bool aligned = rows_aligned(target_logits, V, dt) && (!draft_logits || aligned_to(draft_logits, 16));
    hipStream_t s = (hipStream_t)stream;

    sv::StatsParams sp{};
    sp.target = target_logits;
    sp.draft = draft_logits;
    sp.tokens = draft_tokens;
    sp.lens = draft_lens;
    sp.temp = temperature;
    sp.unif = uniforms;
    sp.B = B; sp.n = n; sp.V = V; sp.NC = L.NC; sp.CH = L.CH; sp.S = S;
    sp.acc = accepted_len;
    sp.emitted = emitted;
    sp.row_lse = row_lse;
    sp.flags = err_flags;
    sp.part = at<sv::Partial>(workspace, L.off_part);
    sp.cnt = at<uint32_t>(workspace, L.off_cnt);
    sp.desc = at<sv::DrawDesc>(workspace, L.off_desc);
    sp.NT = L.NT;
    sp.tiles = at<unsigned long long>(workspace, L.off_tiles);
    sp.R = n + 1;
    sp.row_index = nullptr;
    sp.dstats = draft_stats;
    // no drafts: every draw is a bonus draw, made by the decision (no draw pass)
    sp.draw_in_stats = (SV_DRAW_IN_STATS && n == 0) ? 1 : 0;
    if (mtp && pl.fused) sp.mtp = pl.f;
    hipError_t e = sv::launch_stats(sp, dt == SV_BF16 ? sv::kBF16 : sv::kF32, sv::kSample, aligned, s);
    if (e != hipSuccess) return hip_fail(e);

    if (!sp.draw_in_stats) {
        sv::DrawParams dp{};
        dp.target = target_logits;
        dp.draft = draft_logits;
        dp.B = B; dp.n = n; dp.V = V; dp.NT = L.NT; dp.NCd = L.NCd;
        dp.R = sp.R;
        dp.row_index = sp.row_index;
        dp.tiles = sp.tiles;
        dp.emitted = emitted;
        dp.flags = err_flags;
        dp.desc = sp.desc;
        dp.dsum = at<float>(workspace, L.off_dsum);
        dp.cnt = at<uint32_t>(workspace, L.off_cnt_draw);
        if (mtp && pl.fused) dp.mtp_tokens = pl.f.tokens;
        e = sv::launch_draw(dp, dt == SV_BF16 ? sv::kBF16 : sv::kF32, aligned, s);
        if (e != hipSuccess) return hip_fail(e);
    }
    if (mtp && !pl.fused) {
        e = sv::launch_mtp(pl.sep, pl.sep_aligned, s);
        if (e != hipSuccess) return hip_fail(e);
    }
    return SV_OK;
}

sv_status_t verify_greedy(const void* target_logits, sv_dtype_t dt, const int32_t* draft_tokens,
                          const int32_t* draft_lens, int B, int n, int V, int32_t* accepted_len, int32_t* emitted,
                          uint32_t* err_flags, void* workspace, size_t workspace_bytes, void* stream,
                          const MtpArgs* mtp) {
    if (!valid_sizes(B, n, V) || (dt != SV_F32 && dt != SV_BF16)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target_logits || !draft_lens || !accepted_len || !emitted || (n > 0 && !draft_tokens))
        return SV_EINVAL;
    const size_t es = elem_bytes(dt);
    if (!aligned_to(target_logits, es) || !aligned_to(draft_tokens, 4) || !aligned_to(draft_lens, 4) ||
        !aligned_to(accepted_len, 4) || !aligned_to(emitted, 4) || !aligned_to(err_flags, 4))
        return SV_EALIGN;
    sv::Layout L;
    if (!make_layout(B, n, V, dt, &L)) return SV_EINVAL;
    if (!workspace || workspace_bytes < L.bytes) return SV_EWORKSPACE;
    if (!aligned_to(workspace, 16)) return SV_EALIGN;
    const int S = n + 1;
    if (!grid_ok((long long)B * S * L.NC)) return SV_EINVAL;
    MtpPlan pl{};
    if (mtp) {
        long long elems = 0;
        const sv_status_t ms = check_mtp(*mtp, B, n, &elems);
        if (ms != SV_OK) return ms;
        const Span tok{mtp->tokens, (size_t)B * (n + 1) * 4};
        const Span others[] = {{target_logits, (size_t)B * (n + 1) * V * es},
                               {draft_tokens, (size_t)B * n * 4},
                               {draft_lens, (size_t)B * 4},
                               {accepted_len, (size_t)B * 4},
                               {emitted, (size_t)B * (n + 1) * 4},
                               {err_flags, err_flags ? 4u : 0u},
                               {workspace, workspace_bytes},
                               tok};
        constexpr int kOthers = sizeof(others) / sizeof(others[0]);
        if (overlaps_any(tok, others, kOthers - 1)) return SV_EINVAL;
        if (elems > 0 && overlaps_any(Span{mtp->hdst, (size_t)elems * 2}, others, kOthers)) return SV_EINVAL;
        pl = plan_mtp(*mtp, elems, accepted_len, emitted, B, n);
    }
    hipStream_t s = (hipStream_t)stream;

    sv::StatsParams sp{};
    sp.target = target_logits;
    sp.draft = nullptr;
    sp.tokens = draft_tokens;
    sp.lens = draft_lens;
    sp.B = B; sp.n = n; sp.V = V; sp.NC = L.NC; sp.CH = L.CH; sp.S = S;
    sp.acc = accepted_len;
    sp.emitted = emitted;
    sp.flags = err_flags;
    sp.part = at<sv::Partial>(workspace, L.off_part);
    sp.cnt = at<uint32_t>(workspace, L.off_cnt);
    sp.desc = at<sv::DrawDesc>(workspace, L.off_desc);
    sp.R = n + 1;
    sp.row_index = nullptr;
    if (mtp && pl.fused) sp.mtp = pl.f;
    hipError_t e = sv::launch_stats(sp, dt == SV_BF16 ? sv::kBF16 : sv::kF32, sv::kGreedy,
                                    rows_aligned(target_logits, V, dt), s);
    if (e != hipSuccess) return hip_fail(e);
    if (mtp && !pl.fused) {
        e = sv::launch_mtp(pl.sep, pl.sep_aligned, s);
        if (e != hipSuccess) return hip_fail(e);
    }
    return SV_OK;
}

}  // namespace

namespace sv {

sv_status_t hip_status(hipError_t e) { return hip_fail(e); }

sv_status_t sample_ex(const void* target_logits, const void* draft_logits, sv_dtype_t dt, const int32_t* draft_tokens,
                      const int32_t* draft_lens, const float* temperature, const float* uniforms,
                      const float* draft_stats, int B, int n, int V, int32_t* accepted_len, int32_t* emitted,
                      float* row_lse, uint32_t* err_flags, int32_t* tokens, const void* hidden_src, void* hidden_dst,
                      int H, void* workspace, size_t workspace_bytes, void* stream) {
    if (!tokens && (hidden_src || hidden_dst)) return SV_EINVAL;
    const MtpArgs m{tokens, hidden_src, hidden_dst, H};
    return verify_sample(target_logits, draft_logits, dt, draft_tokens, draft_lens, temperature, uniforms, B, n,
                         V, accepted_len, emitted, row_lse, err_flags, workspace, workspace_bytes, stream,
                         tokens ? &m : nullptr, draft_stats);
}

}  // namespace sv

extern "C" {

sv_status_t spec_verify_sample(const void* target_logits, const void* draft_logits, sv_dtype_t dt,
                               const int32_t* draft_tokens, const int32_t* draft_lens,
                               const float* temperature, const float* uniforms, int B, int n, int V,
                               int32_t* accepted_len, int32_t* emitted, float* row_lse,
                               uint32_t* err_flags, void* workspace, size_t workspace_bytes,
                               void* stream) {
    return verify_sample(target_logits, draft_logits, dt, draft_tokens, draft_lens, temperature, uniforms, B, n,
                         V, accepted_len, emitted, row_lse, err_flags, workspace, workspace_bytes, stream,
                         nullptr, nullptr);
}

sv_status_t spec_verify_sample_mtp(const void* target_logits, const void* draft_logits, sv_dtype_t dt,
                                   const int32_t* draft_tokens, const int32_t* draft_lens,
                                   const float* temperature, const float* uniforms, int B, int n, int V,
                                   int32_t* accepted_len, int32_t* emitted, float* row_lse,
                                   uint32_t* err_flags, int32_t* tokens, const void* hidden_src,
                                   void* hidden_dst, int H, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    const MtpArgs m{tokens, hidden_src, hidden_dst, H};
    return verify_sample(target_logits, draft_logits, dt, draft_tokens, draft_lens, temperature, uniforms, B, n,
                         V, accepted_len, emitted, row_lse, err_flags, workspace, workspace_bytes, stream, &m,
                         nullptr);
}

sv_status_t spec_verify_sample_ex(const void* target_logits, const void* draft_logits, sv_dtype_t dt,
                                  const int32_t* draft_tokens, const int32_t* draft_lens,
                                  const float* temperature, const float* uniforms, const float* draft_stats,
                                  int B, int n, int V, int32_t* accepted_len, int32_t* emitted, float* row_lse,
                                  uint32_t* err_flags, int32_t* tokens, const void* hidden_src,
                                  void* hidden_dst, int H, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    return sv::sample_ex(target_logits, draft_logits, dt, draft_tokens, draft_lens, temperature, uniforms,
                         draft_stats, B, n, V, accepted_len, emitted, row_lse, err_flags, tokens, hidden_src,
                         hidden_dst, H, workspace, workspace_bytes, stream);
}

sv_status_t spec_verify_greedy(const void* target_logits, sv_dtype_t dt, const int32_t* draft_tokens,
                               const int32_t* draft_lens, int B, int n, int V, int32_t* accepted_len,
                               int32_t* emitted, uint32_t* err_flags, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return verify_greedy(target_logits, dt, draft_tokens, draft_lens, B, n, V, accepted_len, emitted, err_flags,
                         workspace, workspace_bytes, stream, nullptr);
}

sv_status_t spec_verify_tree_greedy(const void* target_logits, sv_dtype_t dt, const int32_t* draft_tokens,
                                    const int32_t* draft_parents, const int32_t* draft_lens, int B, int n, int V,
                                    int32_t* accepted_len, int32_t* emitted, int32_t* path, uint32_t* err_flags,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_sizes(B, n, V) || (dt != SV_F32 && dt != SV_BF16)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target_logits || !draft_lens || !accepted_len || !emitted || (n > 0 && (!draft_tokens || !draft_parents)))
        return SV_EINVAL;
    const size_t es = elem_bytes(dt);
    if (!aligned_to(target_logits, es) || !aligned_to(draft_tokens, 4) || !aligned_to(draft_parents, 4) ||
        !aligned_to(draft_lens, 4) || !aligned_to(accepted_len, 4) || !aligned_to(emitted, 4) ||
        !aligned_to(path, 4) || !aligned_to(err_flags, 4))
        return SV_EALIGN;
    sv::Layout L;
    if (!make_layout(B, n, V, dt, &L)) return SV_EINVAL;
    if (!workspace || workspace_bytes < L.bytes) return SV_EWORKSPACE;
    if (!aligned_to(workspace, 16)) return SV_EALIGN;
    const int S = n + 1;
    if (!grid_ok((long long)B * S * L.NC)) return SV_EINVAL;
    sv::StatsParams sp{};
    sp.target = target_logits;
    sp.draft = nullptr;
    sp.tokens = draft_tokens;
    sp.lens = draft_lens;
    sp.B = B; sp.n = n; sp.V = V; sp.NC = L.NC; sp.CH = L.CH; sp.S = S;
    sp.acc = accepted_len;
    sp.emitted = emitted;
    sp.flags = err_flags;
    sp.part = at<sv::Partial>(workspace, L.off_part);
    sp.cnt = at<uint32_t>(workspace, L.off_cnt);
    sp.desc = at<sv::DrawDesc>(workspace, L.off_desc);
    sp.R = n + 1;
    sp.row_index = nullptr;
    sp.parents = draft_parents;
    sp.path = path;
    const hipError_t e = sv::launch_tree(sp, dt == SV_BF16 ? sv::kBF16 : sv::kF32,
                                         rows_aligned(target_logits, V, dt), (hipStream_t)stream);
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

int sv_tree_rounds(const int32_t* parents, int L) {
    if (!parents || L <= 0) return 0;
    if (L > sv::kMaxDraft) L = sv::kMaxDraft;
    int kids[sv::kMaxDraft + 1] = {0}, acc[sv::kMaxDraft + 1] = {0};
    for (int j = 0; j < L; ++j)
        if (parents[j] >= 0 && parents[j] <= j) ++kids[parents[j]];
    // rounds a walk can need at node a: one per rejected child that has a later sibling
    int best = acc[0] = kids[0] > 1 ? kids[0] - 1 : 0;
    for (int i = 1; i <= L; ++i) {
        const int p = parents[i - 1];
        if (!(p >= 0 && p < i)) continue;
        acc[i] = acc[p] + (kids[i] > 1 ? kids[i] - 1 : 0);
        if (acc[i] > best) best = acc[i];
    }
    return best;
}

sv_status_t spec_verify_tree_sample(const void* target_logits, const void* draft_logits, sv_dtype_t dt,
                                    const int32_t* draft_tokens, const int32_t* draft_parents,
                                    const int32_t* draft_lens, const float* temperature, const float* uniforms,
                                    int B, int n, int V, int max_rounds, int32_t* accepted_len, int32_t* emitted,
                                    int32_t* path, uint32_t* err_flags, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    if (!valid_sizes(B, n, V) || (dt != SV_F32 && dt != SV_BF16)) return SV_EINVAL;
    if (max_rounds < 0 || max_rounds > sv::kMaxDraft * sv::kMaxDraft) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target_logits || !draft_lens || !temperature || !uniforms || !accepted_len || !emitted ||
        (n > 0 && (!draft_logits || !draft_tokens || !draft_parents)))
        return SV_EINVAL;
    const size_t es = elem_bytes(dt);
    if (!aligned_to(target_logits, es) || !aligned_to(draft_logits, es) || !aligned_to(draft_tokens, 4) ||
        !aligned_to(draft_parents, 4) || !aligned_to(draft_lens, 4) || !aligned_to(temperature, 4) ||
        !aligned_to(uniforms, 4) || !aligned_to(accepted_len, 4) || !aligned_to(emitted, 4) || !aligned_to(path, 4) ||
        !aligned_to(err_flags, 4))
        return SV_EALIGN;
    sv::Layout L;
    if (!make_layout(B, n, V, dt, &L)) return SV_EINVAL;
    if (!workspace || workspace_bytes < L.bytes) return SV_EWORKSPACE;
    if (!aligned_to(workspace, 16)) return SV_EALIGN;
    const int S = 2 * n + 1;
    if (!grid_ok((long long)B * S * L.NC) || !grid_ok((long long)B * L.NCd)) return SV_EINVAL;
    const bool aligned = rows_aligned(target_logits, V, dt) && aligned_to(draft_logits, 16);
    const sv::Dt kdt = dt == SV_BF16 ? sv::kBF16 : sv::kF32;
    hipStream_t s = (hipStream_t)stream;

    sv::StatsParams sp{};
    sp.target = target_logits;
    sp.draft = draft_logits;
    sp.tokens = draft_tokens;
    sp.lens = draft_lens;
    sp.temp = temperature;
    sp.unif = uniforms;
    sp.B = B; sp.n = n; sp.V = V; sp.NC = L.NC; sp.CH = L.CH; sp.S = S;
    sp.acc = accepted_len;
    sp.emitted = emitted;
    sp.flags = err_flags;
    sp.part = at<sv::Partial>(workspace, L.off_part);
    sp.cnt = at<uint32_t>(workspace, L.off_cnt);
    sp.desc = at<sv::DrawDesc>(workspace, L.off_desc);
    sp.NT = L.NT;
    sp.tiles = at<unsigned long long>(workspace, L.off_tiles);
    sp.R = n + 1;
    sp.parents = draft_parents;
    sp.path = path;
    sp.walk = at<sv::TreeWalk>(workspace, L.off_walk);
    sp.trows = at<char>(workspace, L.off_trows);
    sp.can_pend = max_rounds > 0;
    hipError_t e = sv::launch_tree_sample(sp, kdt, aligned, s);
    if (e != hipSuccess) return hip_fail(e);
    for (int r = 0; r < max_rounds; ++r) {
        sv::RoundParams rp{};
        rp.target = target_logits;
        rp.draft = draft_logits;
        rp.tokens = draft_tokens;
        rp.parents = draft_parents;
        rp.lens = draft_lens;
        rp.unif = uniforms;
        rp.B = B; rp.n = n; rp.V = V; rp.NT = L.NT; rp.NCd = L.NCd;
        rp.walk = sp.walk;
        rp.trows = sp.trows;
        rp.can_pend = r + 1 < max_rounds;
        rp.dsum = at<float>(workspace, L.off_dsum);
        rp.cnt = at<uint32_t>(workspace, L.off_cnt_draw);
        rp.desc = sp.desc;
        rp.acc = accepted_len;
        rp.emitted = emitted;
        rp.path = path;
        rp.flags = err_flags;
        e = sv::launch_tree_round(rp, kdt, aligned, s);
        if (e != hipSuccess) return hip_fail(e);
    }
    sv::DrawParams dp{};
    dp.target = target_logits;
    dp.draft = draft_logits;
    dp.B = B; dp.n = n; dp.V = V; dp.NT = L.NT; dp.NCd = L.NCd;
    dp.R = n + 1;
    dp.row_index = nullptr;
    dp.tiles = sp.tiles;
    dp.emitted = emitted;
    dp.flags = err_flags;
    dp.desc = sp.desc;
    dp.dsum = at<float>(workspace, L.off_dsum);
    dp.cnt = at<uint32_t>(workspace, L.off_cnt_draw);
    e = sv::launch_draw(dp, kdt, aligned, s);
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

sv_status_t spec_verify_greedy_mtp(const void* target_logits, sv_dtype_t dt, const int32_t* draft_tokens,
                                   const int32_t* draft_lens, int B, int n, int V, int32_t* accepted_len,
                                   int32_t* emitted, uint32_t* err_flags, int32_t* tokens,
                                   const void* hidden_src, void* hidden_dst, int H, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    const MtpArgs m{tokens, hidden_src, hidden_dst, H};
    return verify_greedy(target_logits, dt, draft_tokens, draft_lens, B, n, V, accepted_len, emitted, err_flags,
                         workspace, workspace_bytes, stream, &m);
}

sv_status_t sv_sample_rows(const void* logits, sv_dtype_t dt, int R, const int32_t* row_index,
                           const float* temperature, const float* uniforms, int B, int V, int32_t* tokens,
                           uint32_t* err_flags, float* row_stats, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (B < 0 || R < 1 || V < 1 || (dt != SV_F32 && dt != SV_BF16)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!logits || !temperature || !uniforms || !tokens) return SV_EINVAL;
    const size_t es = elem_bytes(dt);
    if (!aligned_to(logits, es) || !aligned_to(row_index, 4) || !aligned_to(temperature, 4) ||
        !aligned_to(uniforms, 4) || !aligned_to(tokens, 4) || !aligned_to(err_flags, 4) ||
        !aligned_to(row_stats, 4))
        return SV_EALIGN;
    sv::Layout L;
    if (!make_layout(B, 0, V, dt, &L)) return SV_EINVAL;
    if (!workspace || workspace_bytes < L.bytes) return SV_EWORKSPACE;
    if (!aligned_to(workspace, 16)) return SV_EALIGN;
    if (!grid_ok((long long)B * L.NC) || !grid_ok((long long)B * L.NCd)) return SV_EINVAL;
    const bool aligned = rows_aligned(logits, V, dt);
    hipStream_t s = (hipStream_t)stream;

    // the verify step with no drafts: one target slot per sequence, row chosen on the device
    sv::StatsParams sp{};
    sp.target = logits;
    sp.draft = nullptr;
    sp.tokens = nullptr;
    sp.lens = nullptr;
    sp.temp = temperature;
    sp.unif = uniforms;
    sp.B = B; sp.n = 0; sp.V = V; sp.NC = L.NC; sp.CH = L.CH; sp.S = 1;
    sp.acc = at<int32_t>(workspace, L.off_acc);
    sp.emitted = tokens;
    sp.row_lse = nullptr;
    sp.flags = err_flags;
    sp.part = at<sv::Partial>(workspace, L.off_part);
    sp.cnt = at<uint32_t>(workspace, L.off_cnt);
    sp.desc = at<sv::DrawDesc>(workspace, L.off_desc);
    sp.NT = L.NT;
    sp.tiles = at<unsigned long long>(workspace, L.off_tiles);
    sp.R = R;
    sp.row_index = row_index;
    sp.out_stats = row_stats;
    sp.draw_in_stats = SV_DRAW_IN_STATS;  // one row per sequence, no drafts: the decision draws
    hipError_t e = sv::launch_stats(sp, dt == SV_BF16 ? sv::kBF16 : sv::kF32, sv::kSample, aligned, s);
    if (e != hipSuccess) return hip_fail(e);
    if (sp.draw_in_stats) return SV_OK;
    sv::DrawParams dp{};
    dp.target = logits;
    dp.draft = nullptr;
    dp.B = B; dp.n = 0; dp.V = V; dp.NT = L.NT; dp.NCd = L.NCd;
    dp.R = R;
    dp.row_index = row_index;
    dp.tiles = sp.tiles;
    dp.emitted = tokens;
    dp.flags = err_flags;
    dp.desc = sp.desc;
    dp.dsum = at<float>(workspace, L.off_dsum);
    dp.cnt = at<uint32_t>(workspace, L.off_cnt_draw);
    e = sv::launch_draw(dp, dt == SV_BF16 ? sv::kBF16 : sv::kF32, aligned, s);
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

sv_status_t mtp_shift_insert(int32_t* tokens, const void* hidden_src, void* hidden_dst, int H,
                             const int32_t* accepted_len, const int32_t* emitted, int B, int n,
                             void* stream) {
    if (B < 0 || n < 0 || n > sv::kMaxDraft || H < 0) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!accepted_len || !emitted) return SV_EINVAL;
    long long elems = 0;
    const sv_status_t ms = check_mtp(MtpArgs{tokens, hidden_src, hidden_dst, H}, B, n, &elems);
    if (ms != SV_OK) return ms;
    if (!aligned_to(accepted_len, 4) || !aligned_to(emitted, 4)) return SV_EALIGN;
    sv::MtpParams mp{};
    mp.tokens = tokens;
    mp.hsrc = hidden_src;
    mp.hdst = hidden_dst;
    mp.hidden_elems = hidden_src ? hidden_elems(B, n, H) : 0;
    mp.acc = accepted_len;
    mp.emitted = emitted;
    mp.B = B;
    mp.n = n;
    const bool aligned = aligned_to(hidden_src, 16) && aligned_to(hidden_dst, 16);
    hipError_t e = sv::launch_mtp(mp, aligned, (hipStream_t)stream);
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// Size checks of the logit projection: H a positive multiple of kLmBK, and the
// 16-byte vector offsets of both matrices within 32 bits.
bool lmhead_sizes_ok(long long M, int H, int V) {
    if (M < 0 || V < 1 || H < sv::kLmBK || H % sv::kLmBK != 0) return false;
    const long long lim = 1ll << 34;  // elements: (elements / 8) vectors < 2^31
    return M * (long long)H < lim && (long long)V * H < lim;
}

}  // namespace

extern "C" {

sv_status_t spec_verify_greedy_lmhead(const void* hidden, const void* weight, int H, const int32_t* draft_tokens,
                                      const int32_t* draft_lens, int B, int n, int V, int32_t* accepted_len,
                                      int32_t* emitted, uint32_t* err_flags, int32_t* tokens, void* hidden_dst,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_sizes(B, n, V)) return SV_EINVAL;
    const long long M = (long long)B * (n + 1);
    if (!lmhead_sizes_ok(M, H, V)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!hidden || !weight || !draft_lens || !accepted_len || !emitted || (n > 0 && !draft_tokens))
        return SV_EINVAL;
    if (!tokens && hidden_dst) return SV_EINVAL;
    if (!aligned_to(hidden, 16) || !aligned_to(weight, 16) || !aligned_to(hidden_dst, 16) ||
        !aligned_to(draft_tokens, 4) || !aligned_to(draft_lens, 4) || !aligned_to(accepted_len, 4) ||
        !aligned_to(emitted, 4) || !aligned_to(err_flags, 4) || !aligned_to(tokens, 4))
        return SV_EALIGN;
    sv::Layout L;
    if (!make_layout(B, n, V, SV_BF16, &L)) return SV_EINVAL;
    if (!workspace || workspace_bytes < L.bytes) return SV_EWORKSPACE;
    if (!aligned_to(workspace, 16)) return SV_EALIGN;
    const size_t hbytes = (size_t)M * H * 2;
    const bool copy = hidden_dst && hidden_dst != hidden;
    if (tokens) {
        const Span tok{tokens, (size_t)M * 4};
        const Span others[] = {{hidden, hbytes},
                               {weight, (size_t)V * H * 2},
                               {draft_tokens, (size_t)B * n * 4},
                               {draft_lens, (size_t)B * 4},
                               {accepted_len, (size_t)B * 4},
                               {emitted, (size_t)M * 4},
                               {err_flags, err_flags ? 4u : 0u},
                               {workspace, workspace_bytes},
                               tok};
        constexpr int kOthers = sizeof(others) / sizeof(others[0]);
        if (overlaps_any(tok, others, kOthers - 1)) return SV_EINVAL;
        if (copy && overlaps_any(Span{hidden_dst, hbytes}, others, kOthers)) return SV_EINVAL;
    }
    hipStream_t s = (hipStream_t)stream;

    // the projection: one argmax key per row, merged into the decision's
    // partial slots (chunk slot 0 of row r of sequence b: b * (n+1) + r)
    sv::LmParams lp{};
    lp.hidden = hidden;
    lp.weight = weight;
    lp.M = (int)M;
    lp.H = H;
    lp.V = V;
    lp.keys = at<unsigned long long>(workspace, L.off_part);
    lp.lens = draft_lens;
    lp.n = n;
    lp.hidden_dst = copy ? hidden_dst : nullptr;
    hipError_t e = sv::launch_lmhead(lp, s);
    if (e != hipSuccess) return hip_fail(e);

    sv::StatsParams sp{};
    sp.tokens = draft_tokens;
    sp.lens = draft_lens;
    sp.B = B; sp.n = n; sp.V = V; sp.NC = 1; sp.CH = V; sp.S = n + 1;
    sp.acc = accepted_len;
    sp.emitted = emitted;
    sp.flags = err_flags;
    sp.part = at<sv::Partial>(workspace, L.off_part);
    sp.cnt = at<uint32_t>(workspace, L.off_cnt);
    sp.desc = at<sv::DrawDesc>(workspace, L.off_desc);
    sp.R = n + 1;
    sp.row_index = nullptr;
    sp.mtp.tokens = tokens;
    e = sv::launch_decide_greedy(sp, s);
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

sv_status_t sv_lmhead_logits_debug(const void* hidden, const void* weight, int M, int H, int V, float* logits_out,
                                   void* stream) {
    if (!lmhead_sizes_ok(M, H, V)) return SV_EINVAL;
    if (M == 0) return SV_OK;
    if (!hidden || !weight || !logits_out) return SV_EINVAL;
    if (!aligned_to(hidden, 16) || !aligned_to(weight, 16) || !aligned_to(logits_out, 4)) return SV_EALIGN;
    sv::LmParams lp{};
    lp.hidden = hidden;
    lp.weight = weight;
    lp.M = M;
    lp.H = H;
    lp.V = V;
    lp.logits = logits_out;
    hipError_t e = sv::launch_lmhead(lp, (hipStream_t)stream);
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

sv_status_t sv_softmax_rows_debug(const void* logits, sv_dtype_t dt, const float* temperature, int rows,
                                  int V, float* probs_out, void* stream) {
    if (rows < 0 || V < 1 || (dt != SV_F32 && dt != SV_BF16)) return SV_EINVAL;
    if (rows == 0) return SV_OK;
    if (!logits || !temperature || !probs_out) return SV_EINVAL;
    if (!aligned_to(logits, elem_bytes(dt)) || !aligned_to(temperature, 4) || !aligned_to(probs_out, 4))
        return SV_EALIGN;
    hipError_t e = sv::launch_softmax_debug(logits, dt == SV_BF16 ? sv::kBF16 : sv::kF32, temperature, rows,
                                            V, probs_out, rows_aligned(logits, V, dt), (hipStream_t)stream);
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

sv_status_t sv_residual_weights_debug(const void* target_rows, const void* draft_rows, sv_dtype_t dt,
                                      const float* temperature, int rows, int V, float* weights_out,
                                      double* tile_weights_out, float* info_out, void* stream) {
    if (rows < 0 || V < 1 || (dt != SV_F32 && dt != SV_BF16)) return SV_EINVAL;
    if (rows == 0) return SV_OK;
    if (!target_rows || !draft_rows || !temperature || !weights_out) return SV_EINVAL;
    const size_t es = elem_bytes(dt);
    if (!aligned_to(target_rows, es) || !aligned_to(draft_rows, es) || !aligned_to(temperature, 4) ||
        !aligned_to(weights_out, 4) || !aligned_to(tile_weights_out, 8) || !aligned_to(info_out, 4))
        return SV_EALIGN;
    sv::Layout L;
    if (!make_layout(1, 0, V, dt, &L)) return SV_EINVAL;
    const bool aligned = rows_aligned(target_rows, V, dt) && aligned_to(draft_rows, 16);
    hipError_t e = sv::launch_residual_debug(target_rows, draft_rows, dt == SV_BF16 ? sv::kBF16 : sv::kF32,
                                             temperature, rows, V, L.NT, weights_out, tile_weights_out, info_out,
                                             aligned, (hipStream_t)stream);
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

}  // extern "C"
