// Host side of libgdn: argument validation, workspace layout and launch
// order for the C ABI declared in include/gdn.h. Every check runs before the
// first HIP call, so a rejected call enqueues nothing and the checks can be
// exercised without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

using gdn::BT;
using gdn::DK;
using gdn::DV;

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;   // sanity bound on any tensor

// _packed_offsets rules (hyper-parallel Diff Coverage page): at least two
// entries, first 0, last total, strictly increasing.
bool offsets_ok(const int32_t* offs, int32_t n, int64_t total) {
    if (offs == nullptr || n < 2) return false;
    if (offs[0] != 0 || offs[n - 1] != total) return false;
    for (int32_t i = 0; i + 1 < n; ++i)
        if (offs[i] >= offs[i + 1]) return false;
    return true;
}

int64_t count_chunks(const int32_t* offs, int32_t n, int32_t cs) {
    int64_t c = 0;
    for (int32_t i = 0; i + 1 < n; ++i) c += (int64_t(offs[i + 1]) - offs[i] + cs - 1) / cs;
    return c;
}

gdn_status validate(const gdn_desc* d, gdn::Problem* p) {
    if (d == nullptr) return GDN_ERR_INVALID;
    if (d->chunk_size != 64) return GDN_ERR_INVALID;
    if (d->K != DK || d->V != DV) return GDN_ERR_UNSUPPORTED;
    if (d->B < 1 || d->T < 0 || d->H < 1) return GDN_ERR_INVALID;
    if (d->layout != GDN_LAYOUT_BSND && d->layout != GDN_LAYOUT_TND) return GDN_ERR_INVALID;
    if (d->dtype != GDN_DTYPE_F32 && d->dtype != GDN_DTYPE_BF16) return GDN_ERR_INVALID;
    if (d->o_dtype != GDN_DTYPE_F32 && d->o_dtype != GDN_DTYPE_BF16) return GDN_ERR_INVALID;
    if (d->gate_kind != GDN_GATE_SCALAR && d->gate_kind != GDN_GATE_PER_KEY) return GDN_ERR_INVALID;
    if (d->use_exp2 != 0 && d->use_exp2 != 1) return GDN_ERR_INVALID;
    if (!isfinite(d->scale)) return GDN_ERR_INVALID;
    const int64_t total = int64_t(d->B) * d->T;
    if (total * d->H * DK > kMaxElems) return GDN_ERR_INVALID;
    p->reorder = 0;
    p->qk_norm = 0;
    p->beta_sig = 0;
    gdn::UnitMap um;
    memset(&um, 0, sizeof(um));
    um.T = d->T;
    um.row_stride = d->T;
    um.t_base = 0;
    um.total_tokens = total;
    if (d->layout == GDN_LAYOUT_TND) {
        // packed documents: physical batch one, offsets required
        if (d->B != 1 || d->n_units < 1) return GDN_ERR_INVALID;
    }
    if (d->n_units < 0) return GDN_ERR_INVALID;
    if (d->n_units == 0) {
        um.dense = 1;
        um.n_units = d->B;
        um.nt_dense = (d->T + BT - 1) / BT;
        const int64_t nc = int64_t(d->B) * um.nt_dense;
        if (nc > INT32_MAX / 2) return GDN_ERR_INVALID;
        um.n_chunks = (int32_t)nc;
    } else {
        if (!offsets_ok(d->offsets_host, d->n_units + 1, total)) return GDN_ERR_INVALID;
        if (d->layout == GDN_LAYOUT_BSND) {
            // segments of rows: every row start must be a unit boundary
            int32_t j = 0;
            for (int32_t b = 1; b < d->B; ++b) {
                const int64_t rs = int64_t(b) * d->T;
                while (j <= d->n_units && d->offsets_host[j] < rs) ++j;
                if (j > d->n_units || d->offsets_host[j] != rs) return GDN_ERR_INVALID;
            }
        }
        if (!d->offsets_dev || !d->chunk_offsets_dev || !d->chunk_indices_dev) return GDN_ERR_INVALID;
        const int64_t nc = count_chunks(d->offsets_host, d->n_units + 1, BT);
        if (nc > INT32_MAX / 2) return GDN_ERR_INVALID;
        um.dense = 0;
        um.n_units = d->n_units;
        um.n_chunks = (int32_t)nc;
        um.offsets = d->offsets_dev;
        um.chunk_offsets = d->chunk_offsets_dev;
        um.chunk_indices = d->chunk_indices_dev;
        // the state passes launch the units longest first unless they already
        // come in non-increasing chunk count
        for (int32_t u = 1; u < d->n_units && !p->reorder; ++u) {
            const int64_t a = (int64_t(d->offsets_host[u]) - d->offsets_host[u - 1] + BT - 1) / BT;
            const int64_t b = (int64_t(d->offsets_host[u + 1]) - d->offsets_host[u] + BT - 1) / BT;
            p->reorder = b > a;
        }
    }
    p->H = d->H;
    p->dtype = d->dtype;
    p->o_dtype = d->o_dtype;
    p->per_key = d->gate_kind == GDN_GATE_PER_KEY;
    p->use_exp2 = d->use_exp2;
    p->scale = d->scale;
    p->um = um;
    return GDN_OK;
}

gdn_status size_workspace(const gdn::Problem& p, void* workspace, size_t* workspace_bytes,
                          gdn::Workspace* ws, bool* query_only) {
    if (workspace_bytes == nullptr) return GDN_ERR_INVALID;
    const size_t need = gdn::workspace_bytes(p, nullptr, nullptr);
    *query_only = workspace == nullptr;
    if (workspace == nullptr) {
        *workspace_bytes = need;
        return GDN_OK;
    }
    if (*workspace_bytes < need) {
        *workspace_bytes = need;
        return GDN_ERR_CAPACITY;
    }
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return GDN_ERR_INVALID;
    gdn::workspace_bytes(p, ws, static_cast<char*>(workspace));
    return GDN_OK;
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

}  // namespace

// Workspace layout: regions 256-byte aligned, one slot per (chunk, head) in
// chunk-major order. With ws and base given, also sets the region pointers.
size_t gdn::workspace_bytes(const gdn::Problem& p, gdn::Workspace* ws, char* base) {
    const int64_t nch = (int64_t)p.um.n_chunks * p.H;
    const int64_t es = p.dtype == 1 ? 2 : 4;      // operand element size (fp16 or fp32)
    int64_t off = 0;
    auto take = [&](int64_t bytes) { int64_t o = off; off = align256(off + bytes); return o; };
    const int64_t oT = take(nch * BT * BT * es);
    const int64_t oP = take(nch * BT * BT * es);
    const int64_t og = (p.dtype == 0 && !p.per_key) ? take(nch * GAMR * BT * 4) : 0;
    int64_t oq = 0, od = 0, ok = 0, ol = 0;
    if (p.per_key) {
        oq = take(nch * BT * DK * es);
        od = take(nch * BT * DK * es);
        ok = take(nch * BT * DK * es);
        ol = take(nch * DK * 4);
    }
    const int64_t ocf = p.dtype == 1 ? take(nch * (p.per_key ? CFB : CFS)) : 0;
    const bool ordered = p.reorder && !p.um.dense && p.um.n_units > 1 && p.um.n_units <= ORD_MAX;
    const int64_t oor = ordered ? take((int64_t)p.um.n_units * 4) : 0;
    if (ws && base) {
        ws->Tm = base + oT;
        ws->P = base + oP;
        ws->gam = (p.dtype == 0 && !p.per_key) ? reinterpret_cast<float*>(base + og) : nullptr;
        ws->qg = p.per_key ? base + oq : nullptr;
        ws->kd = p.per_key ? base + od : nullptr;
        ws->kg = p.per_key ? base + ok : nullptr;
        ws->gamL = p.per_key ? reinterpret_cast<float*>(base + ol) : nullptr;
        ws->cfh = p.dtype == 1 ? base + ocf : nullptr;
        ws->order = ordered ? reinterpret_cast<int32_t*>(base + oor) : nullptr;
    }
    return (size_t)(off > 0 ? off : 256);
}


extern "C" gdn_status gdn_varlen_meta(const int32_t* offsets, int32_t n_offsets, int32_t total_tokens,
                                      int32_t chunk_size, int32_t* chunk_indices, int32_t cap_chunks,
                                      int32_t* chunk_offsets, int32_t* n_chunks_out) {
    if (chunk_size <= 0 || total_tokens < 1) return GDN_ERR_INVALID;
    if (!offsets_ok(offsets, n_offsets, total_tokens)) return GDN_ERR_INVALID;
    const int64_t nc = count_chunks(offsets, n_offsets, chunk_size);
    if (nc > INT32_MAX) return GDN_ERR_INVALID;
    if (n_chunks_out) *n_chunks_out = (int32_t)nc;
    if (chunk_offsets) {
        int64_t c = 0;
        for (int32_t i = 0; i + 1 < n_offsets; ++i) {
            chunk_offsets[i] = (int32_t)c;
            c += (int64_t(offsets[i + 1]) - offsets[i] + chunk_size - 1) / chunk_size;
        }
        chunk_offsets[n_offsets - 1] = (int32_t)c;
    }
    if (chunk_indices) {
        if (cap_chunks < nc) return GDN_ERR_CAPACITY;
        int64_t c = 0;
        for (int32_t i = 0; i + 1 < n_offsets; ++i) {
            const int64_t m = (int64_t(offsets[i + 1]) - offsets[i] + chunk_size - 1) / chunk_size;
            for (int64_t j = 0; j < m; ++j, ++c) {
                chunk_indices[2 * c] = i;
                chunk_indices[2 * c + 1] = (int32_t)j;
            }
        }
    }
    return GDN_OK;
}

// Every check of gdn_chunk_fwd that does not involve the workspace.
gdn_status gdn::fwd_preflight(const gdn_desc* desc, const void* q, const void* k, const void* v,
                              const float* g, const void* beta, const void* o, int32_t flags,
                              gdn::Problem* p, size_t* workspace_need) {
    gdn_status st = validate(desc, p);
    if (st != GDN_OK) return st;
    if (flags & ~(GDN_FLAG_REUSE_PREPARED | GDN_FLAG_PREPARE_ONLY | GDN_FLAG_QK_L2NORM | GDN_FLAG_BETA_SIGMOID))
        return GDN_ERR_INVALID;
    const bool reuse = flags & GDN_FLAG_REUSE_PREPARED, prep_only = flags & GDN_FLAG_PREPARE_ONLY;
    if (reuse && prep_only) return GDN_ERR_INVALID;
    p->qk_norm = (flags & GDN_FLAG_QK_L2NORM) != 0;
    p->beta_sig = (flags & GDN_FLAG_BETA_SIGMOID) != 0;
    const bool tokens = p->um.total_tokens > 0;
    if (tokens && (!k || !g || !beta)) return GDN_ERR_INVALID;
    if (!prep_only && tokens && (!q || !v || !o)) return GDN_ERR_INVALID;
    if (p->per_key && !reuse && tokens && !q) return GDN_ERR_INVALID;   // the per-key preparation gates q
    if (workspace_need) *workspace_need = gdn::workspace_bytes(*p, nullptr, nullptr);
    return GDN_OK;
}

// ---- the forward in pieces
// Dense rows so few that the state pass leaves most of the GPU idle (at most
// 128 workgroups) and long enough to cut: the forward runs over pieces of
// consecutive chunks of every row. The preparation of every piece is issued
// on a helper stream, the state pass of piece i on the caller's stream after
// the preparation of piece i, from the state piece i - 1 left; so the
// preparation of later pieces runs beside the state pass of earlier ones.
// The pieces' preparations and the state between pieces take their own
// workspace regions.
namespace {

constexpr int kPipeMaxPieces = 8;

int pipe_pieces(const gdn::Problem& p) {
    if (!p.um.dense) return 0;
    if (int64_t(p.um.n_units) * p.H * (DV / 32) > 128) return 0;
    if (p.um.nt_dense < 128) return 0;
    const int n = p.um.nt_dense / 64;
    return n < kPipeMaxPieces ? n : kPipeMaxPieces;
}

gdn::Problem pipe_piece(const gdn::Problem& p, int i, int n) {
    const int per = (p.um.nt_dense + n - 1) / n;
    const int c0 = i * per, c1 = (c0 + per < p.um.nt_dense) ? c0 + per : p.um.nt_dense;
    gdn::Problem q = p;
    const int64_t t0 = int64_t(c0) * BT, t1 = int64_t(c1) * BT < p.um.T ? int64_t(c1) * BT : p.um.T;
    q.um.t_base = p.um.t_base + t0;
    q.um.T = (int32_t)(t1 - t0);
    q.um.nt_dense = c1 - c0;
    q.um.n_chunks = p.um.n_units * (c1 - c0);
    return q;
}

// workspace of the pieces, then the state between them (fp32 [units][H][K][V])
size_t pipe_workspace(const gdn::Problem& p, int n, gdn::Workspace* ws, float** carry, char* base) {
    size_t off = 0;
    for (int i = 0; i < n; ++i) {
        const gdn::Problem q = pipe_piece(p, i, n);
        const size_t b = gdn::workspace_bytes(q, nullptr, nullptr);
        if (ws && base) gdn::workspace_bytes(q, &ws[i], base + off);
        off += (b + 255) & ~size_t(255);
    }
    if (carry && base) *carry = reinterpret_cast<float*>(base + off);
    off += size_t(p.um.n_units) * p.H * DK * DV * 4;
    return off;
}

struct PipeStreams {
    hipStream_t aux = nullptr;
    hipEvent_t start = nullptr;
    hipEvent_t prepared[kPipeMaxPieces] = {};
    bool ready = false;
};
PipeStreams g_pipe[64];
std::mutex g_pipe_mu;

// the helper stream and events of the current device, made on first use;
// NULL (the caller then runs the single pass) when they cannot be made,
// when the caller's stream belongs to another device (whose helper stream
// would have to be made with that device current), or when the stream is
// being captured into a graph (the single pass keeps the graph on the
// caller's stream, with no stream made during the capture)
PipeStreams* pipe_streams(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    if (stream) {
        hipDevice_t sdev = 0;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return nullptr;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    }
    PipeStreams& ps = g_pipe[dev];
    if (!ps.ready) {
        if (hipStreamCreateWithFlags(&ps.aux, hipStreamNonBlocking) != hipSuccess) return nullptr;
        if (hipEventCreateWithFlags(&ps.start, hipEventDisableTiming) != hipSuccess) return nullptr;
        for (auto& e : ps.prepared)
            if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
        ps.ready = true;
    }
    return &ps;
}

}  // namespace

extern "C" gdn_status gdn_chunk_fwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                    const float* g, const void* beta, const float* initial_state,
                                    void* o, float* final_state, const gdn_slots* slots, int32_t flags,
                                    void* workspace, size_t* workspace_bytes, hipStream_t stream) {
    return gdn::fwd_impl(desc, q, k, v, g, beta, initial_state, o, final_state, slots, flags, workspace,
                         workspace_bytes, stream, true);
}

gdn_status gdn::fwd_impl(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                         const void* beta, const float* initial_state, void* o, float* final_state,
                         const gdn_slots* slots, int32_t flags, void* workspace, size_t* workspace_bytes,
                         hipStream_t stream, bool allow_pipeline) {
    gdn::Problem p;
    gdn_status st = validate(desc, &p);
    if (st != GDN_OK) return st;
    // pipelined problems keep room for their pieces (the single pass fits in it too)
    const int pieces = allow_pipeline ? pipe_pieces(p) : 0;
    if (pieces > 0) {
        if (workspace_bytes == nullptr) return GDN_ERR_INVALID;
        const size_t need = pipe_workspace(p, pieces, nullptr, nullptr, nullptr);
        if (workspace == nullptr) {
            *workspace_bytes = need;
            return GDN_OK;
        }
        if (*workspace_bytes < need) {
            *workspace_bytes = need;
            return GDN_ERR_CAPACITY;
        }
    }
    gdn::Workspace ws;
    bool query = false;
    st = size_workspace(p, workspace, workspace_bytes, &ws, &query);
    if (st != GDN_OK || query) return st;
    st = gdn::fwd_preflight(desc, q, k, v, g, beta, o, flags, &p, nullptr);
    if (st != GDN_OK) return st;
    const bool reuse = flags & GDN_FLAG_REUSE_PREPARED, prep_only = flags & GDN_FLAG_PREPARE_ONLY;
    if (pieces > 0 && !reuse && !prep_only && !(slots && slots->h) && p.um.total_tokens > 0) {
        gdn::PrepSlots ps = {};
        if (slots) {
            ps.g_cumsum = slots->g_cumsum;
            ps.A = slots->A;
            ps.q_hat = slots->q_hat;
            ps.k_hat = slots->k_hat;
            ps.q_rstd = slots->q_rstd;
            ps.k_rstd = slots->k_rstd;
            ps.beta_eff = slots->beta_eff;
        }
        std::lock_guard<std::mutex> lock(g_pipe_mu);
        PipeStreams* pst = pipe_streams(stream);
        if (pst) {
            gdn::Workspace pws[kPipeMaxPieces];
            float* carry = nullptr;
            pipe_workspace(p, pieces, pws, &carry, static_cast<char*>(workspace));
            if (final_state) carry = final_state;   // each workgroup reads its tile before it writes it
            if (hipEventRecord(pst->start, stream) != hipSuccess) return GDN_ERR_DEVICE;
            if (hipStreamWaitEvent(pst->aux, pst->start, 0) != hipSuccess) return GDN_ERR_DEVICE;
            for (int i = 0; i < pieces; ++i) {
                // the first preparation has the GPU to itself
                if (gdn::launch_prep(pipe_piece(p, i, pieces), pws[i], k, q, g, beta, ps, pst->aux, i > 0) != hipSuccess)
                    return GDN_ERR_DEVICE;
                if (hipEventRecord(pst->prepared[i], pst->aux) != hipSuccess) return GDN_ERR_DEVICE;
            }
            for (int i = 0; i < pieces; ++i) {
                if (hipStreamWaitEvent(stream, pst->prepared[i], 0) != hipSuccess) return GDN_ERR_DEVICE;
                const float* h0 = i == 0 ? initial_state : carry;
                float* hf = i + 1 < pieces ? carry : final_state;
                if (gdn::launch_state(pipe_piece(p, i, pieces), pws[i], q, k, v, beta, h0, o, hf, nullptr,
                                      slots ? slots->v_new : nullptr, 0, 0, 0, nullptr, nullptr, nullptr, 0,
                                      stream) != hipSuccess)
                    return GDN_ERR_DEVICE;
            }
            return GDN_OK;
        }
    }
    gdn::PrepSlots ps = {};
    if (slots) {
        ps.g_cumsum = slots->g_cumsum;
        ps.A = slots->A;
        ps.q_hat = slots->q_hat;
        ps.k_hat = slots->k_hat;
        ps.q_rstd = slots->q_rstd;
        ps.k_rstd = slots->k_rstd;
        ps.beta_eff = slots->beta_eff;
    }
    // q_hat and q_rstd come from q, which a preparation without q does not read
    if (!q && (ps.q_hat || ps.q_rstd)) return GDN_ERR_INVALID;
    if (!reuse) {
        if (gdn::launch_prep(p, ws, k, q, g, beta, ps, stream) != hipSuccess) return GDN_ERR_DEVICE;
    }
    if (!prep_only) {
        if (gdn::launch_state(p, ws, q, k, v, beta, initial_state, o, final_state, slots ? slots->h : nullptr,
                              slots ? slots->v_new : nullptr, 0, 0, 0, nullptr, nullptr, nullptr, 0,
                              stream) != hipSuccess)
            return GDN_ERR_DEVICE;
    }
    return GDN_OK;
}

extern "C" gdn_status gdn_state_summary(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                        const float* g, const void* beta, int32_t mode, int32_t flags,
                                        const int32_t* units_dev, int32_t n_sel, float* S_ext, float* M,
                                        void* workspace, size_t* workspace_bytes, hipStream_t stream) {
    gdn::Problem p;
    gdn_status st = validate(desc, &p);
    if (st != GDN_OK) return st;
    if (mode < 0 || mode > 2) return GDN_ERR_INVALID;
    if (flags & ~(GDN_FLAG_REUSE_PREPARED | GDN_FLAG_QK_L2NORM | GDN_FLAG_BETA_SIGMOID)) return GDN_ERR_INVALID;
    p.qk_norm = (flags & GDN_FLAG_QK_L2NORM) != 0;
    p.beta_sig = (flags & GDN_FLAG_BETA_SIGMOID) != 0;
    const bool all = n_sel < 0;
    if (n_sel > p.um.n_units || (n_sel > 0 && !units_dev)) return GDN_ERR_INVALID;
    const bool want_ext = mode != 2, want_M = mode != 1;
    gdn::Workspace ws;
    bool query = false;
    st = size_workspace(p, workspace, workspace_bytes, &ws, &query);
    if (st != GDN_OK || query) return st;
    if ((want_ext && !S_ext) || (want_M && !M)) return GDN_ERR_INVALID;
    const bool tokens = p.um.total_tokens > 0;
    if (tokens && (!k || !v || !g || !beta)) return GDN_ERR_INVALID;
    if (!(flags & GDN_FLAG_REUSE_PREPARED) &&
        gdn::launch_prep(p, ws, k, q, g, beta, gdn::PrepSlots{}, stream) != hipSuccess)
        return GDN_ERR_DEVICE;
    if (n_sel == 0) return GDN_OK;
    if (gdn::launch_state(p, ws, nullptr, k, v, beta, nullptr, nullptr, nullptr, nullptr, nullptr, 1, want_ext,
                          want_M, S_ext, M, all ? nullptr : units_dev, n_sel, stream) != hipSuccess)
        return GDN_ERR_DEVICE;
    return GDN_OK;
}

extern "C" gdn_status gdn_split_meta(const int32_t* doc_offsets, int32_t n_doc_offsets, const int32_t* seg_offsets,
                                     int32_t n_seg_offsets, int32_t total_tokens, int32_t* piece_offsets,
                                     int32_t* piece_doc, int32_t* piece_seg, int32_t cap_pieces,
                                     int32_t* n_pieces_out) {
    if (total_tokens < 1) return GDN_ERR_INVALID;
    if (!offsets_ok(doc_offsets, n_doc_offsets, total_tokens)) return GDN_ERR_INVALID;
    if (!offsets_ok(seg_offsets, n_seg_offsets, total_tokens)) return GDN_ERR_INVALID;
    // the pieces are the gaps of the merged, de-duplicated cut lists
    int32_t i = 1, j = 1, n = 0, d = 0, sgi = 0, start = 0;
    while (i < n_doc_offsets || j < n_seg_offsets) {
        const int32_t a = i < n_doc_offsets ? doc_offsets[i] : INT32_MAX;
        const int32_t b = j < n_seg_offsets ? seg_offsets[j] : INT32_MAX;
        const int32_t end = a < b ? a : b;
        if (piece_offsets && n < cap_pieces) {
            piece_offsets[n] = start;
            piece_offsets[n + 1] = end;
            if (piece_doc) piece_doc[n] = d;
            if (piece_seg) piece_seg[n] = sgi;
        }
        ++n;
        if (a == end) { ++i; ++d; }
        if (b == end) { ++j; ++sgi; }
        start = end;
    }
    if (n_pieces_out) *n_pieces_out = n;
    if (piece_offsets && cap_pieces < n) return GDN_ERR_CAPACITY;
    return GDN_OK;
}

extern "C" gdn_status gdn_state_merge_pieces(int32_t n_pieces, int32_t n_docs, int32_t H, int32_t K, int32_t V,
                                             const int32_t* piece_doc_dev, const float* S_ext, const float* M,
                                             const float* S0_docs, float* S_in, hipStream_t stream) {
    if (K != DK || V != DV) return GDN_ERR_UNSUPPORTED;
    if (n_pieces < 0 || n_docs < 1 || H < 1 || n_docs > (1 << 26) || H > 65535) return GDN_ERR_INVALID;
    if (int64_t(n_pieces) * H * DK * DK > kMaxElems) return GDN_ERR_INVALID;
    if (n_pieces > 0 && (!piece_doc_dev || !S_ext || !M || !S_in)) return GDN_ERR_INVALID;
    if (gdn::launch_merge_pieces(n_pieces, n_docs, H, piece_doc_dev, S_ext, M, S0_docs, S_in, stream) != hipSuccess)
        return GDN_ERR_DEVICE;
    return GDN_OK;
}

// Workspace of the backward: the preparation (T, P and the gate rows of every
// chunk-head; per key, the gated q and k tiles and G_last, fp32), then dL/dh
// at every chunk's exit and dvn of every chunk (fp32 regions; the bf16
// scalar-gate path keeps fp16 values and its chunk maps in them; per key the
// second region holds the fp32 chunk maps A of the state gradient instead).
static size_t bwd_workspace(const gdn::Problem& p, gdn::Workspace* ws, float** dH, float** dVN, char* base) {
    gdn::Problem pf = p;
    pf.dtype = 0;
    pf.reorder = 0;
    const int64_t prep = (int64_t)gdn::workspace_bytes(pf, ws, base);
    const int64_t nch = (int64_t)p.um.n_chunks * p.H;
    const int64_t o1 = align256(prep), o2 = align256(o1 + nch * DK * DV * 4);
    // per key: the chunk maps A of the state gradient (fp32 K x K) in place
    // of dvn, which the per-key gradient kernel forms itself
    const int64_t end = align256(o2 + (p.per_key ? nch * DK * DK * 4 : nch * BT * DV * 4));
    if (base) {
        *dH = reinterpret_cast<float*>(base + o1);
        *dVN = reinterpret_cast<float*>(base + o2);
    }
    return (size_t)end;
}

extern "C" gdn_status gdn_chunk_bwd(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                    const float* g, const void* beta, const float* h, const void* dout,
                                    const float* dht, float* dq, float* dk, float* dv, float* dg,
                                    float* dbeta, float* dh0, int32_t flags, void* workspace,
                                    size_t* workspace_bytes, hipStream_t stream) {
    gdn::Problem p;
    gdn_status st = validate(desc, &p);
    if (st != GDN_OK) return st;
    if (flags != 0 && flags != GDN_FLAG_REUSE_PREPARED) return GDN_ERR_INVALID;
    if (workspace_bytes == nullptr) return GDN_ERR_INVALID;
    const size_t need = bwd_workspace(p, nullptr, nullptr, nullptr, nullptr);
    if (workspace == nullptr) {
        *workspace_bytes = need;
        return GDN_OK;
    }
    if (*workspace_bytes < need) {
        *workspace_bytes = need;
        return GDN_ERR_CAPACITY;
    }
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return GDN_ERR_INVALID;
    const bool tokens = p.um.total_tokens > 0;
    if (tokens && (!q || !k || !v || !g || !beta || !h || !dout || !dq || !dk || !dv || !dg || !dbeta))
        return GDN_ERR_INVALID;
    gdn::Workspace ws;
    float *dH = nullptr, *dVN = nullptr;
    bwd_workspace(p, &ws, &dH, &dVN, static_cast<char*>(workspace));
    if (gdn::launch_bwd(p, ws, dH, dVN, q, k, v, g, beta, h, dout, dht, dq, dk, dv, dg, dbeta, dh0, false,
                        flags == GDN_FLAG_REUSE_PREPARED, stream) != hipSuccess)
        return GDN_ERR_DEVICE;
    return GDN_OK;
}

extern "C" gdn_status gdn_state_grad_summary(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                             const float* g, const void* beta, const float* h, const void* dout,
                                             float* dS_ext, int32_t flags, void* workspace,
                                             size_t* workspace_bytes, hipStream_t stream) {
    gdn::Problem p;
    gdn_status st = validate(desc, &p);
    if (st != GDN_OK) return st;
    if (flags != 0 && flags != GDN_FLAG_REUSE_PREPARED) return GDN_ERR_INVALID;
    if (workspace_bytes == nullptr) return GDN_ERR_INVALID;
    const size_t need = bwd_workspace(p, nullptr, nullptr, nullptr, nullptr);
    if (workspace == nullptr) {
        *workspace_bytes = need;
        return GDN_OK;
    }
    if (*workspace_bytes < need) {
        *workspace_bytes = need;
        return GDN_ERR_CAPACITY;
    }
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return GDN_ERR_INVALID;
    if (!dS_ext) return GDN_ERR_INVALID;
    if (p.um.total_tokens > 0 && (!q || !k || !v || !g || !beta || !h || !dout)) return GDN_ERR_INVALID;
    gdn::Workspace ws;
    float *dH = nullptr, *dVN = nullptr;
    bwd_workspace(p, &ws, &dH, &dVN, static_cast<char*>(workspace));
    if (gdn::launch_bwd(p, ws, dH, dVN, q, k, v, g, beta, h, dout, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, dS_ext, true, flags == GDN_FLAG_REUSE_PREPARED, stream) != hipSuccess)
        return GDN_ERR_DEVICE;
    return GDN_OK;
}

extern "C" gdn_status gdn_state_merge_adjoint(int32_t B, int32_t H, int32_t n_seg, int32_t K, int32_t V,
                                              const float* dS_ext, const float* M, const float* dS_final,
                                              float* dS_exit, float* dS0, hipStream_t stream) {
    if (K != DK || V != DV) return GDN_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || n_seg < 0) return GDN_ERR_INVALID;
    if (int64_t(B) * H * n_seg * DK * DK > kMaxElems) return GDN_ERR_INVALID;
    if (n_seg > 0 && (!dS_ext || !M || !dS_exit)) return GDN_ERR_INVALID;
    if (gdn::launch_merge_adjoint(B, H, n_seg, dS_ext, M, dS_final, dS_exit, dS0, stream) != hipSuccess)
        return GDN_ERR_DEVICE;
    return GDN_OK;
}

extern "C" gdn_status gdn_state_merge(int32_t B, int32_t H, int32_t n_seg, int32_t K, int32_t V,
                                      const float* S_ext, const float* M, const float* S0, float* S_init,
                                      float* S_final, hipStream_t stream) {
    if (K != DK || V != DV) return GDN_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || n_seg < 0) return GDN_ERR_INVALID;
    if (int64_t(B) * H * n_seg * DK * DK > kMaxElems) return GDN_ERR_INVALID;
    if (n_seg > 0 && (!S_ext || !M || !S_init)) return GDN_ERR_INVALID;
    if (gdn::launch_merge(B, H, n_seg, S_ext, M, S0, S_init, S_final, stream) != hipSuccess)
        return GDN_ERR_DEVICE;
    return GDN_OK;
}
