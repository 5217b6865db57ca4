// HIP kernels of the chunked gated delta rule backward (scalar and per-key
// gates) for gfx950.
//
// The forward of one chunk (n <= 64 tokens, entry state h in K x V, G the
// chunk-local inclusive cumulative gate, b the decay base, gamma = b^{G_L}):
//   Kd = diag(b^G) K, Qd = diag(b^G) Q, Kg = diag(b^{G_L - G}) K
//   L  = strict_tril(diag(beta) (K K^T o D)),  D_ij = b^{G_i - G_j}
//   T  = (I + L)^{-1},  Tb = T diag(beta)
//   Y  = V - Kd h,  v_new = Tb Y
//   O  = scale (Qd h + P v_new),  P = tril(Q K^T o D)
//   h' = gamma h + Kg^T v_new
// Given dO and dh' = dL/dh', reverse mode gives
//   dvn = scale P^T dO + Kg dh'          Z = Tb^T dvn
//   dh  = gamma dh' + scale Qd^T dO - Kd^T Z          (the reverse state pass)
//   dV  = Z,  dKd = -Z h^T,  dQd = scale dO h^T,  dKg = v_new dh'^T
//   dP  = scale dO v_new^T,  dTb = dvn Y^T,  dT = dTb diag(beta)
//   dL  = -T^T dT T^T (strictly lower),  dbeta_j += sum_i dTb_ij T_ij,
//   dbeta_i += sum_j dL_ij (k_i.k_j) D_ij
// then dk, dq and the cumulative-gate gradient dG from the D factors, Kd, Qd,
// Kg and gamma, and dg as the reverse cumulative sum of dG inside the chunk.
// These are the stages of the staged backward on the hyper-parallel Diff
// Coverage page (_AscendCKDAStages.backward: prepare, the reverse state pass
// chunk_gated_delta_rule_bwd_dhu, finalize) and the reverse chunk loop of
// kda_state_grad_ext_kernel on the state_summary.py page (the state gradient
// decays by b^{G_L}, then gains Q^T dO scale - W^T (value gradient)).
//
// Every barrier is an LDS hand-off (lds_barrier): no thread reads global
// memory that another thread of the kernel writes, so the per-chunk stores
// (dh', dvn, dv) stay in flight across barriers.
//
// Kernels:
//   bwd_dh_kernel    one workgroup per (unit, head, 16 or 32 value columns):
//                    the reverse state pass; stores dh' and dvn of every
//                    chunk and dL/dS0.
//   bwd_grad_kernel  one workgroup per (chunk, head): recomputes Y and v_new
//                    from the stored entry state, accumulates the products
//                    over the value columns in tiles, then forms dq, dk, dv,
//                    dbeta and dg.
// fp32 inputs and the per-key gate use fp32 operands (fp32 16x16x4 MFMA,
// fp32 LDS tiles) and the fp32 preparation (T, P, gate rows or gated tiles).
// bf16 inputs with a scalar gate use bwd_dh_kernel_h and bwd_grad_kernel_h:
// fp16 LDS tiles and the fp16 16x16x32 MFMA with fp32 accumulation, fed by
// the forward's bf16 preparation writing T and P as fp16.
//
// Per-key gate (b^G a 64 x K matrix): Kd, Qd and Kg are the prepared gated
// tiles and gamma = diag(b^{G_L}), so the reverse state pass and the value-
// tile products are the same with those tiles in place of the row scalings.
// The decay inside L and P is per key, D_ijd = b^{G_id - G_jd}; with
// X = dL (strictly lower) and dP (lower with the diagonal) the finish needs
//   R[X, Y]_id = sum_j X_ij Y_jd D_ijd      (rows)
//   C[X, Y]_jd = sum_i X_ij Y_id D_ijd      (columns)
// for R[dL, K], R[dP, K], C[diag(beta) dL, K] and C[dP, Q]:
//   dq = R[dP,K] + b^G o dQd
//   dk = beta o R[dL,K] + C[beta dL,K] + C[dP,Q] + b^G o dKd + b^{G_L-G} o dKg
//   dG = ln b (beta k o R[dL,K] + q o R[dP,K] - k o (C[beta dL,K] + C[dP,Q])
//              + Qd o dQd + Kd o dKd - Kg o dKg),   dbeta_i += k_i . R[dL,K]_i
// and G_L gains ln b (sum_i Kg o dKg + gamma o diag(h dh'^T)). Since dg is
// the reverse sum of dG inside the chunk with G_L's gradient at the last
// row, the two Kg o dKg parts cancel for every row from i on; both gates
// therefore compute dg_j = sum_{i >= j} dG_i (without the Kg part) + ln b
// gamma o diag(h dh'^T) + sum_{i < j} ln b Kg_i o dKg_i, which keeps the
// cancellation out of the rounding (the scalar gate's rows are the same
// with one key). Off the
// diagonal 16-row blocks each product splits the decay at a reference row r
// between the two blocks, b^{G_i - G_r} b^{G_r - G_j}, both factors at most 1
// for any g <= 0 (the forward's preparation does the same for L and P); the
// diagonal blocks take the exponent differences directly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int BKL = DK + 4;     // row stride (floats) of the 64 x 128 k and q tiles
constexpr int BTL = BT + 1;     // row stride of the 64 x 64 T, P and scratch tiles

struct BwdArgs {
    UnitMap um;
    int H;
    int use_exp2;
    float scale;
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    const float* g;        // per key: the gates (the finish rebuilds G in key slices)
    const void* dout;
    const float* h;        // [n_chunks][H][K][V] entry state of every chunk
    const float* dht;      // [units][H][K][V] or NULL
    float* dq;
    float* dk;
    float* dv;
    float* dg;
    float* dbeta;
    float* dh0;            // [units][H][K][V] or NULL
    Workspace ws;          // fp32 preparation: T, P, gate rows
    float* dH;             // [n_chunks][H][K][V]  dL/dh at every chunk's exit
    float* dVN;            // [n_chunks][H][64][V] dvn of every chunk
    int n_pairs;
};

template <class In>
__device__ __forceinline__ float ldf(const In* p, int64_t i) { return (float)p[i]; }

// acc += A B on the fp32 16x16x4 MFMA over k in [0, KLEN): lane (G, n)
// supplies A[n][k0 + G] = fa(n, k0 + G) and B[k0 + G][n] = fb(k0 + G, n) and
// holds D[4G + r][n]
template <int KLEN, class FA, class FB>
__device__ __forceinline__ void mmf(f32x4& acc, FA fa, FB fb, int G, int n) {
#pragma unroll 8
    for (int k0 = 0; k0 < KLEN; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa(n, k0 + G), fb(k0 + G, n), acc, 0, 0, 0);
}

// 16 bytes of inputs -> fp32 (4 fp32 or 8 bf16 values)
template <class In> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ static void cvt(u32x4 w, float* x) { for (int i = 0; i < 4; ++i) x[i] = u2f(w[i]); }
};
template <> struct Vec16<f16> {
    static constexpr int N = 8;
    __device__ static void cvt(u32x4 w, float* x) {
        const f16x8 h = __builtin_bit_cast(f16x8, w);
        for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
    }
};
template <> struct Vec16<bf16> {
    static constexpr int N = 8;
    __device__ static void cvt(u32x4 w, float* x) {
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = u2f(w[i] << 16);
            x[2 * i + 1] = u2f(w[i] & 0xffff0000u);
        }
    }
};

// ROWS x NCOLS elements of a tile (row r at src + r * stride, rows at or
// past `valid` read as zero) as 16-byte vectors in registers: issue() loads
// them, commit() converts them to fp32 and stores them into an LDS tile with
// row stride ld (optionally scaling column c by scale[c % 4], the four
// columns every vector of a thread covers when NCOLS is 4 VPR * 16). Between
// the two the vectors may stay in flight.
template <class In, int ROWS, int NCOLS>
struct TileRegs {
    static constexpr int VPR = Vec16<In>::N, PER_ROW = NCOLS / VPR, NV = ROWS * PER_ROW;
    static constexpr int PT = (NV + 255) / 256;
    u32x4 w[PT];
    __device__ __forceinline__ void issue(const In* src, int64_t stride, int valid, int tid) {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int e = tid + 256 * i, r = e / PER_ROW, c = (e - r * PER_ROW) * VPR;
            w[i] = u32x4{0u, 0u, 0u, 0u};
            if (e < NV && r < valid) w[i] = *reinterpret_cast<const u32x4*>(src + r * stride + c);
        }
    }
    __device__ __forceinline__ void commit(float* dst, int ld, int tid, const float* colscale = nullptr) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int e = tid + 256 * i, r = e / PER_ROW, c = (e - r * PER_ROW) * VPR;
            if (e < NV) {
                float x[VPR];
                Vec16<In>::cvt(w[i], x);
                for (int j = 0; j < VPR; ++j) dst[r * ld + c + j] = colscale ? x[j] * colscale[j % 4] : x[j];
            }
        }
    }
    // the same, transposed: element (r, c) to dst[c * ld + r]
    __device__ __forceinline__ void commit_tr(float* dst, int ld, int tid) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int e = tid + 256 * i, r = e / PER_ROW, c = (e - r * PER_ROW) * VPR;
            if (e < NV) {
                float x[VPR];
                Vec16<In>::cvt(w[i], x);
                for (int j = 0; j < VPR; ++j) dst[(c + j) * ld + r] = x[j];
            }
        }
    }
    // the same, as fp16 values (8 bytes per fp32 vector, 16 per bf16 or fp16
    // one), and with column c + j of a vector scaled by colscale[j] into dst2
    // when given
    __device__ __forceinline__ void commit_h(f16* dst, int ld, int tid, const float* colscale = nullptr,
                                             f16* dst2 = nullptr) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int e = tid + 256 * i, r = e / PER_ROW, c = (e - r * PER_ROW) * VPR;
            if (e < NV) {
                float x[VPR];
                Vec16<In>::cvt(w[i], x);
                typedef _Float16 hv __attribute__((ext_vector_type(VPR)));
                hv h;
                for (int j = 0; j < VPR; ++j) h[j] = (f16)x[j];
                *reinterpret_cast<hv*>(dst + r * ld + c) = h;
                if (dst2) {
                    for (int j = 0; j < VPR; ++j) h[j] = (f16)(x[j] * colscale[j]);
                    *reinterpret_cast<hv*>(dst2 + r * ld + c) = h;
                }
            }
        }
    }
    // fp16 values scaled by s (one row per thread: PT == 1)
    __device__ __forceinline__ void commit_h_mul(f16* dst, int ld, int tid, float s) const {
        static_assert(PT == 1, "one vector per thread");
        const int e = tid, r = e / PER_ROW, c = (e - r * PER_ROW) * VPR;
        if (e < NV) {
            float x[VPR];
            Vec16<In>::cvt(w[0], x);
            typedef _Float16 hv __attribute__((ext_vector_type(VPR)));
            hv h;
            for (int j = 0; j < VPR; ++j) h[j] = (f16)(x[j] * s);
            *reinterpret_cast<hv*>(dst + r * ld + c) = h;
        }
    }
    // fp16 values with vector i's row scaled by rowscale[i]
    __device__ __forceinline__ void commit_h_rows(f16* dst, int ld, int tid, const float* rowscale) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int e = tid + 256 * i, r = e / PER_ROW, c = (e - r * PER_ROW) * VPR;
            if (e < NV) {
                float x[VPR];
                Vec16<In>::cvt(w[i], x);
                typedef _Float16 hv __attribute__((ext_vector_type(VPR)));
                hv h;
                for (int j = 0; j < VPR; ++j) h[j] = (f16)(x[j] * rowscale[i]);
                *reinterpret_cast<hv*>(dst + r * ld + c) = h;
            }
        }
    }
    // the 16-byte vectors as they are (fp16 tiles)
    __device__ __forceinline__ void commit_raw(f16* dst, int ld, int tid) const {
        static_assert(std::is_same<In, f16>::value, "raw copies of fp16 tiles");
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int e = tid + 256 * i, r = e / PER_ROW, c = (e - r * PER_ROW) * VPR;
            if (e < NV) *reinterpret_cast<u32x4*>(dst + r * ld + c) = w[i];
        }
    }
    // fp16 values with column c + j of a vector scaled by colscale[j]
    __device__ __forceinline__ void commit_h_cols(f16* dst, int ld, int tid, const float* colscale) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int e = tid + 256 * i, r = e / PER_ROW, c = (e - r * PER_ROW) * VPR;
            if (e < NV) {
                float x[VPR];
                Vec16<In>::cvt(w[i], x);
                typedef _Float16 hv __attribute__((ext_vector_type(VPR)));
                hv h;
                for (int j = 0; j < VPR; ++j) h[j] = (f16)(x[j] * colscale[j]);
                *reinterpret_cast<hv*>(dst + r * ld + c) = h;
            }
        }
    }
};

// a tile into LDS: all loads issued before any store, so that their
// latencies overlap
template <class In, int ROWS, int NCOLS>
__device__ __forceinline__ void load_tile(const In* src, int64_t stride, int valid, float* dst, int ld, int tid) {
    TileRegs<In, ROWS, NCOLS> t;
    t.issue(src, stride, valid, tid);
    t.commit(dst, ld, tid);
}

// the chunk's k and q tiles, T (or T diag(beta)), P, the gate rows and beta
template <class In, bool TB>
__device__ void load_chunk(const BwdArgs& a, int64_t t0, int64_t ch, int head, int len, float* Ks, float* Qs,
                           float* Ts, float* Ps, float* gm, float* bt, int tid) {
    const int64_t rs = (int64_t)a.H * DK;
    load_tile<In, BT, DK>(reinterpret_cast<const In*>(a.k) + (t0 * a.H + head) * DK, rs, len, Ks, BKL, tid);
    load_tile<In, BT, DK>(reinterpret_cast<const In*>(a.q) + (t0 * a.H + head) * DK, rs, len, Qs, BKL, tid);
    load_tile<float, BT, BT>(reinterpret_cast<const float*>(a.ws.Tm) + ch * (BT * BT), BT, BT, Ts, BTL, tid);
    load_tile<float, BT, BT>(reinterpret_cast<const float*>(a.ws.P) + ch * (BT * BT), BT, BT, Ps, BTL, tid);
    if (tid < BT) bt[tid] = tid < len ? ldf(reinterpret_cast<const In*>(a.beta), (t0 + tid) * a.H + head) : 0.0f;
    gm[tid] = a.ws.gam[ch * (GAMR * BT) + tid];   // rows 0..3 (the backward has no q / k normalisation)
    lds_barrier();
    if (TB)
        for (int e = tid; e < BT * BT; e += 256) Ts[(e >> 6) * BTL + (e & 63)] *= bt[e & 63];
}

}  // namespace

// acc += A B^T over k in [0, KLEN), A and B stored row by row with k
// contiguous (rows lda / ldb floats apart, 16-byte aligned): lane (G, n)
// reads k = k0 + 4G .. +3 of row n of each with one 16-byte load per 16 k,
// as four fp32 MFMAs
template <int KLEN>
__device__ __forceinline__ void mm_rowsk(f32x4& acc, const float* A, int lda, const float* B, int ldb, int G, int n) {
#pragma unroll
    for (int k0 = 0; k0 < KLEN; k0 += 16) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(A + n * lda + k0 + 4 * G);
        const f32x4 y = *reinterpret_cast<const f32x4*>(B + n * ldb + k0 + 4 * G);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e], y[e], acc, 0, 0, 0);
    }
}

// ------------------------------------------------------------------ reverse state pass
// fp32 inputs with a scalar gate (fp32 operands; the per-key gate takes the
// affine form below). One workgroup of four waves per (unit, head, 16 NCT
// value columns); wave w
// holds dL/dh for keys 32w .. 32w+31 of those columns (2 NCT 16 x 16 tiles).
// NCT = 1 (16-column tiles) doubles the workgroups where 32-column tiles
// would leave compute units idle.
// Chunks run from the last: store dh', then dvn = Kg dh' + scale P^T dO (wave
// w: token rows 16w .. +15), Z = Tb^T dvn, and dh = gamma dh' + scale Qd^T dO
// - Kd^T Z.
template <int NCT>
__global__ __launch_bounds__(256) void bwd_dh_kernel(BwdArgs a) {
    using In = float;
    constexpr int NC = 16 * NCT, CL = NC + 1;   // columns of the tile, LDS row stride
    __shared__ __attribute__((aligned(16))) float Ks[BT * BKL];
    __shared__ __attribute__((aligned(16))) float Qs[BT * BKL];
    __shared__ __attribute__((aligned(16))) float Ts[BT * BTL];     // T diag(beta)
    __shared__ __attribute__((aligned(16))) float Ps[BT * BTL];
    __shared__ __attribute__((aligned(16))) float gm[4 * BT];       // G, b^G, b^{G_L - G}, b^{G_L}
    __shared__ float bt[BT];
    __shared__ __attribute__((aligned(16))) float dOs[BT * CL];     // dO of the tile's columns
    __shared__ __attribute__((aligned(16))) float dhT[NC * BKL];    // dh' [column][key]
    __shared__ __attribute__((aligned(16))) float dvS[BT * CL];     // dvn
    __shared__ __attribute__((aligned(16))) float Zs[BT * CL];      // b^G Z

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H;
    // XCD-aware: workgroups are dealt to the 8 XCDs round-robin, so the
    // column tiles of one (unit, head), which read the same chunk tiles, are
    // given grid slots 8 apart and share that XCD's L2
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int tile = slot % (DV / NC), pair = (slot / (DV / NC)) * 8 + xcd;
    if (pair >= a.n_pairs) return;
    const int u = pair / H, head = pair - u * H;
    const UnitInfo ui = uniform(unit_info(a.um, u));
    const int c0 = tile * NC;
    const int64_t uh = (int64_t)u * H + head;
    const In* dout = reinterpret_cast<const In*>(a.dout);

    // dL/dh at the unit's end: keys 32w + 16kt + 4G + r, column c0 + 16ct + n
    f32x4 dh[2][NCT];
    for (int kt = 0; kt < 2; ++kt)
        for (int ct = 0; ct < NCT; ++ct)
            for (int r = 0; r < 4; ++r) {
                const int key = 32 * w + 16 * kt + 4 * G + r, col = 16 * ct + n;
                const float x = a.dht ? a.dht[(uh * DK + key) * DV + c0 + col] : 0.0f;
                dh[kt][ct][r] = x;
                dhT[col * BKL + key] = x;
            }


    for (int c = ui.nch - 1; c >= 0; --c) {
        int len = ui.len - c * BT;
        len = len > BT ? BT : len;
        const int64_t t0 = ui.start + (int64_t)c * BT;
        const int64_t ch = (int64_t)(ui.cbase + c) * H + head;
        lds_barrier();                               // the previous chunk's tiles are consumed
        load_chunk<In, true>(a, t0, ch, head, len, Ks, Qs, Ts, Ps, gm, bt, tid);
        load_tile<In, BT, NC>(dout + (t0 * H + head) * DV + c0, (int64_t)H * DV, len, dOs, CL, tid);
        // dh' of this chunk to the workspace
        for (int kt = 0; kt < 2; ++kt)
            for (int ct = 0; ct < NCT; ++ct)
                for (int r = 0; r < 4; ++r) {
                    const int key = 32 * w + 16 * kt + 4 * G + r;
                    a.dH[(ch * DK + key) * DV + c0 + 16 * ct + n] = dh[kt][ct][r];
                }
        lds_barrier();
        // dvn = Kg dh' + scale P^T dO, token rows 16w .. +15, with
        // Kg = diag(b^{G_L - G}) K
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 kh = {0.f, 0.f, 0.f, 0.f}, pd = {0.f, 0.f, 0.f, 0.f};
            mm_rowsk<DK>(kh, Ks + 16 * w * BKL, BKL, dhT + 16 * ct * BKL, BKL, G, n);
            mmf<BT>(pd, [&](int m, int k) { return Ps[k * BTL + 16 * w + m]; },
                    [&](int k, int nn) { return dOs[k * CL + 16 * ct + nn]; }, G, n);
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * w + 4 * G + r;
                const float x = gm[2 * BT + row] * kh[r] + a.scale * pd[r];
                dvS[row * CL + 16 * ct + n] = x;
                a.dVN[(ch * BT + row) * DV + c0 + 16 * ct + n] = x;
            }
        }
        lds_barrier();
        // Z = Tb^T dvn, kept as b^G Z
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            mmf<BT>(z, [&](int m, int k) { return Ts[k * BTL + 16 * w + m]; },
                    [&](int k, int nn) { return dvS[k * CL + 16 * ct + nn]; }, G, n);
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * w + 4 * G + r;
                Zs[row * CL + 16 * ct + n] = gm[BT + row] * z[r];
            }
        }
        lds_barrier();
        // dh = gamma dh' + Qd^T (scale dO) - Kd^T Z, keys 32w .. +31, as
        // Q^T (scale b^G dO) - K^T (b^G Z)
        const float gam = gm[3 * BT];
        for (int kt = 0; kt < 2; ++kt)
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acz = {0.f, 0.f, 0.f, 0.f};
                const int key0 = 32 * w + 16 * kt;
                mmf<BT>(acc, [&](int m, int k) { return Qs[k * BKL + key0 + m]; },
                        [&](int k, int nn) { return a.scale * gm[BT + k] * dOs[k * CL + 16 * ct + nn]; },
                        G, n);
                mmf<BT>(acz, [&](int m, int k) { return Ks[k * BKL + key0 + m]; },
                        [&](int k, int nn) { return Zs[k * CL + 16 * ct + nn]; }, G, n);
                for (int r = 0; r < 4; ++r) dh[kt][ct][r] = gam * dh[kt][ct][r] + acc[r] - acz[r];
                // keys key0 + 4G .. +3 of column 16 ct + n: one 16-byte store
                *reinterpret_cast<f32x4*>(&dhT[(16 * ct + n) * BKL + key0 + 4 * G]) = dh[kt][ct];
            }
    }
    if (a.dh0)
        for (int kt = 0; kt < 2; ++kt)
            for (int ct = 0; ct < NCT; ++ct)
                for (int r = 0; r < 4; ++r) {
                    const int key = 32 * w + 16 * kt + 4 * G + r;
                    a.dh0[(uh * DK + key) * DV + c0 + 16 * ct + n] = dh[kt][ct][r];
                }
}

// ------------------------------------------------------------------ per-chunk gradients
// fp32 operands: fp32 inputs with a scalar gate (bwd_grad_kernel), and the
// per-key gate at either input dtype (bwd_grad_kernel_pk, eight waves). The
// value columns are visited in 16-column tiles: each recomputes
// Y = V - Kd h and v_new = Tb Y, writes dV = Z = Tb^T dvn, and accumulates
// over its columns dP, dTb (64 x 64) and dQd, dKg, dKd (64 x 128) in
// registers. The finish turns dTb into dL through T, and assembles dq, dk,
// dbeta and the gate gradients. In bwd_grad_kernel one workgroup of four
// waves per (chunk, head); wave w owns token rows 16w .. 16w+15 of every
// row-indexed product.
constexpr int VT = 16;          // value columns per tile
constexpr int VTL = VT + 4;     // row stride: 16-byte aligned rows; rows 80 bytes apart hit distinct granules

// acc += A B^T over the 16 value columns of a tile, both operands stored row
// by row with the columns contiguous: lane (G, n) reads columns 4G .. 4G+3 of
// row n of each with one 16-byte load, and MFMA e contracts column 4G' + e
// of every lane group G' (the order of the terms inside one contraction
// does not matter)
__device__ __forceinline__ void mm_rows16(f32x4& acc, const float* A, const float* B, float sa, int G, int n) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(A + n * VTL + 4 * G);
    const f32x4 y = *reinterpret_cast<const f32x4*>(B + n * VTL + 4 * G);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sa * x[e], y[e], acc, 0, 0, 0);
}

// The per-key finish of bwd_grad_kernel_pk. On entry: dl = dL of this wave's
// rows (negated) for column blocks 2 grp, 2 grp + 1, X2 = dP (lower with the
// diagonal), dbT = the column term of dbeta, aQ / aKd / aKg = the wave's
// dQd / dKd / dKg tiles in accumulator layout (rows row0 + 4G + r, key tile
// 2s + grp of slice s), hk = per-thread shares of diag(h dh'^T). Ks and Qs
// are free: the key slices (k, q, G, dG of 32 keys) live in Qs, the per-key
// sums in Ks. Wave w8 takes token block w = w8 & 3 and the key tile
// grp = w8 >> 2 of every slice, for both the row and the column products;
// the two groups' dbeta row terms meet in brs.
template <class In>
__device__ __forceinline__ void finish_per_key8(const BwdArgs& a, int64_t t0, int head, int len, int row0, int w,
                                                int w8, int grp, int G, int n, int lane, int tid, const f32x4* dl,
                                                const f32x4* aQ, const f32x4* aKd, const f32x4* aKg, float* hk,
                                                float* X1, const float* X2, float* Ks, float* Qs, const float* bt,
                                                const float* dbT, float* brs) {
    constexpr int SL = 33;                       // row stride of the slice tiles
    const int H = a.H, ue = a.use_exp2;
    const float lnb = ue ? 0.6931471805599453f : 1.0f;
    float* Ksl = Qs;
    float* Qsl = Qs + BT * SL;
    float* Gsl = Qs + 2 * BT * SL;
    float* dGs = Qs + 3 * BT * SL;
    float* hdK = Ks;                             // [DK] diag(h dh'^T)
    float* KGs = Ks + DK;                        // [BT][SL] ln b Kg o dKg of the slice
    float* blk = KGs + BT * SL;                  // [4][64] the waves' block totals of the dg sums
    const In* kin = reinterpret_cast<const In*>(a.k);
    const In* qin = reinterpret_cast<const In*>(a.q);
    const int last = len > 0 ? len - 1 : 0;

    // dL into X1 (strictly lower); diag(h dh'^T) per key over the 16 columns
    // of each thread group
    for (int jh = 0; jh < 2; ++jh)
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + 4 * G + r, jj = 16 * (2 * grp + jh) + n;
            X1[i * BTL + jj] = jj < i ? -dl[jh][r] : 0.0f;
        }
    for (int m = 0; m < 4; ++m) {
        float x = hk[m];
        for (int sft = 1; sft < 16; sft <<= 1) x += __shfl_xor(x, sft, 16);
        if ((tid & 15) == 0) hdK[(tid >> 4) + 32 * m] = x;
    }
    float brow[4] = {0.f, 0.f, 0.f, 0.f};        // k_i . R[dL,K]_i over this lane's keys
    // the key slices' k, q and g tiles, one slice ahead
    TileRegs<In, BT, 32> pk, pq;
    TileRegs<float, BT, 32> pg;
    auto issue = [&](int d0) {
        if (tid >= 256) return;
        pk.issue(kin + (t0 * H + head) * DK + d0, (int64_t)H * DK, len, tid);
        pq.issue(qin + (t0 * H + head) * DK + d0, (int64_t)H * DK, len, tid);
        pg.issue(a.g + (t0 * H + head) * DK + d0, (int64_t)H * DK, len, tid);
    };
    issue(0);

    // the slice loop stays rolled (its body is large); the slice's two key
    // tiles of dQd / dKd / dKg are picked out of the register arrays first
#pragma unroll 1
    for (int s = 0; s < DK / 32; ++s) {
        const int d0 = 32 * s;
        f32x4 sQ, sKd, sKg;                      // this group's key tile of the slice
        switch (s) {
#define GDN_PICK(S)                                                \
    case S:                                                        \
        sQ = aQ[S]; sKd = aKd[S]; sKg = aKg[S];                    \
        break;
            GDN_PICK(0) GDN_PICK(1) GDN_PICK(2) default: GDN_PICK(3)
#undef GDN_PICK
        }
        lds_barrier();                         // X1 written; the previous slice consumed
        if (tid < 256) {
            pk.commit(Ksl, SL, tid);
            pq.commit(Qsl, SL, tid);
            pg.commit(Gsl, SL, tid);
        }
        if (s + 1 < DK / 32) issue(d0 + 32);
        lds_barrier();
        // G: running sum down each key column (rows past the chunk end keep G
        // at its last row) in fp64, rounded once, as the preparation does:
        // lane l of wave 0 sums column l & 31 over rows 32 (l >> 5) .. +31,
        // the upper half from the lower half's total
        if (w8 == 0) {
            const int c = lane & 31, r0 = 32 * (lane >> 5);
            float gv[32];
#pragma unroll
            for (int r = 0; r < 32; ++r) gv[r] = Gsl[(r0 + r) * SL + c];
            double half = 0.0;
#pragma unroll
            for (int r = 0; r < 32; ++r) half += (double)gv[r];
            const double lo = __shfl(half, c, 64);
            double x = lane >= 32 ? lo : 0.0;
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                x += (double)gv[r];
                Gsl[(r0 + r) * SL + c] = (float)x;
            }
        }
        lds_barrier();
        {
            const int c = 16 * grp + n;          // slice column of this lane's key (the group's key tile)
            f32x4 ra = {0.f, 0.f, 0.f, 0.f}, rp = ra, ca = ra, cp = ra;
            // The diagonal block joins the factored products below when the
            // gate falls by at most 2^8 of decay (8 log2 units) inside the
            // block on every key of the tile: its factors about the reference
            // rows then stay within 2^8 (the forward preparation's rule).
            // The stored zeros of dL (strictly lower) and dP (lower with the
            // diagonal) mask the terms past the diagonal.
            const float g_lo = w > 0 ? Gsl[(16 * w - 1) * SL + c] : 0.0f;
            const bool fdiag = __all(g_lo - Gsl[(16 * w + 15) * SL + c] <= (ue ? 8.0f : 5.545177444479562f));
            // rows of block w against the earlier blocks (and the diagonal
            // block when factored): reference row 16w - 1, the last one
            // before the block (the chunk start, G = 0, for block 0)
            const int rend = 16 * w + (fdiag ? 16 : 0);
            if (rend > 0) {
                const float gr = g_lo;
                for (int k0 = 0; k0 < rend; k0 += 4) {
                    const int j = k0 + G;
                    const float b = Ksl[j * SL + c] * fpow(gr - Gsl[j * SL + c], ue);
                    ra = __builtin_amdgcn_mfma_f32_16x16x4f32(X1[(row0 + n) * BTL + j], b, ra, 0, 0, 0);
                    rp = __builtin_amdgcn_mfma_f32_16x16x4f32(X2[(row0 + n) * BTL + j], b, rp, 0, 0, 0);
                }
                for (int r = 0; r < 4; ++r) {
                    const float f = fpow(Gsl[(row0 + 4 * G + r) * SL + c] - gr, ue);
                    ra[r] *= f;
                    rp[r] *= f;
                }
            }
            // columns of block w against the later blocks (and the diagonal
            // block when factored): reference row 16w + 15, the block's last
            const int cbeg = 16 * w + (fdiag ? 0 : 16);
            if (cbeg < BT) {
                const int ref = 16 * w + 15;
                const float gr = Gsl[ref * SL + c];
                for (int k0 = cbeg; k0 < BT; k0 += 4) {
                    const int i = k0 + G;
                    const float f = fpow(Gsl[i * SL + c] - gr, ue);
                    ca = __builtin_amdgcn_mfma_f32_16x16x4f32(bt[i] * X1[i * BTL + row0 + n], Ksl[i * SL + c] * f, ca,
                                                             0, 0, 0);
                    cp = __builtin_amdgcn_mfma_f32_16x16x4f32(X2[i * BTL + row0 + n], Qsl[i * SL + c] * f, cp, 0, 0, 0);
                }
                for (int r = 0; r < 4; ++r) {
                    const float f = fpow(gr - Gsl[(row0 + 4 * G + r) * SL + c], ue);
                    ca[r] *= f;
                    cp[r] *= f;
                }
            }
            // otherwise the diagonal block by exponent differences: m <= i
            // feeds the row products of row i, m >= i the column products of
            // column i; row m's g, k, q and beta are read once for the lane's
            // four rows
            if (!fdiag) {
                float gi[4];
                for (int r = 0; r < 4; ++r) gi[r] = Gsl[(row0 + 4 * G + r) * SL + c];
#pragma unroll 4
                for (int m = row0; m < row0 + 16; ++m) {
                    const float gmv = Gsl[m * SL + c], kmv = Ksl[m * SL + c], qmv = Qsl[m * SL + c], bmv = bt[m];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = row0 + 4 * G + r;
                        const float dd = fpow(m <= i ? gi[r] - gmv : gmv - gi[r], ue);
                        const float km = kmv * dd;
                        if (m <= i) {
                            ra[r] += X1[i * BTL + m] * km;
                            rp[r] += X2[i * BTL + m] * km;
                        }
                        if (m >= i) {
                            ca[r] += bmv * X1[m * BTL + i] * km;
                            cp[r] += X2[m * BTL + i] * qmv * dd;
                        }
                    }
                }
            }
            // gradients of this lane's rows and key
            for (int r = 0; r < 4; ++r) {
                const int i = row0 + 4 * G + r;
                const float gi = Gsl[i * SL + c];
                const float e1 = fpow(gi, ue), e2 = fpow(Gsl[last * SL + c] - gi, ue);
                const float qv = Qsl[i * SL + c], kv = Ksl[i * SL + c];
                const float dQd = sQ[r], dKd = sKd[r], dKg = sKg[r];
                const float cs = ca[r] + cp[r];
                const float dqv = rp[r] + dQd * e1;
                const float dkv = bt[i] * ra[r] + cs + dKd * e1 + dKg * e2;
                // the Kg term of dG_i without its - ln b Kg o dKg: that part
                // cancels G_L's + ln b Kg o dKg for every row from i on and
                // enters dg as the prefix over the earlier rows (below)
                dGs[i * SL + c] = lnb * (bt[i] * kv * ra[r] + qv * rp[r] - kv * cs + dQd * qv * e1 + dKd * kv * e1);
                KGs[i * SL + c] = lnb * dKg * kv * e2;
                brow[r] += kv * ra[r];
                if (i < len) {
                    const int64_t o = ((t0 + i) * H + head) * DK + d0 + c;
                    a.dq[o] = dqv;
                    a.dk[o] = dkv;
                }
            }
        }
        lds_barrier();
        // dg_j = sum_{i >= j} dG_i + ln b gamma diag(h dh'^T) + sum_{i < j}
        // ln b Kg o dKg: a reverse sum down each key column (the state
        // decay's term at the last valid row) and the exclusive prefix of the
        // Kg terms. Waves w (reverse sums) and w + 4 (prefixes) sum rows
        // 16w .. +15 of every column in order on lanes 0..31, then start from
        // the other row blocks' totals.
        {
            const int c = lane & 31;
            const bool rev = grp == 0, act = lane < 32;
            const float gl = rev ? lnb * fpow(Gsl[last * SL + c], ue) * hdK[d0 + c] : 0.0f;
            float v[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 16 * w + r;
                const float x = rev ? dGs[row * SL + c] + (row == last ? gl : 0.0f) : KGs[row * SL + c];
                v[r] = row < len ? x : 0.0f;
            }
            float tot = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) tot += v[r];
            if (act) blk[(4 * grp + w) * 32 + c] = tot;
            lds_barrier();
            float acc = 0.0f;
            for (int w2 = 0; w2 < 4; ++w2)
                if (rev ? w2 > w : w2 < w) acc += blk[(4 * grp + w2) * 32 + c];
            if (act && rev) {
#pragma unroll
                for (int r = 15; r >= 0; --r) {
                    acc += v[r];
                    dGs[(16 * w + r) * SL + c] = acc;
                }
            } else if (act) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    KGs[(16 * w + r) * SL + c] = acc;
                    acc += v[r];
                }
            }
        }
        lds_barrier();
        for (int e = tid; e < BT * 32; e += 512) {
            const int r = e >> 5, c = e & 31;
            if (r < len) a.dg[((t0 + r) * H + head) * DK + d0 + c] = dGs[r * SL + c] + KGs[r * SL + c];
        }
    }
    // dbeta: the row term summed over the 16 lanes of each group, added to the
    // column term of the same row (each row has one writer)
    for (int r = 0; r < 4; ++r)
        for (int sft = 1; sft < 16; sft <<= 1) brow[r] += __shfl_xor(brow[r], sft, 16);
    if (n == 0)
        for (int r = 0; r < 4; ++r) brs[grp * BT + row0 + 4 * G + r] = brow[r];
    lds_barrier();
    if (tid < len) a.dbeta[(t0 + tid) * H + head] = dbT[tid] + brs[tid] + brs[BT + tid];
}

__global__ __launch_bounds__(256) void bwd_grad_kernel(BwdArgs a) {
    using In = float;
    __shared__ __attribute__((aligned(16))) float Ks[BT * BKL];
    __shared__ __attribute__((aligned(16))) float Qs[BT * BKL];
    __shared__ __attribute__((aligned(16))) float Ts[BT * BTL];     // T
    __shared__ __attribute__((aligned(16))) float Ps[BT * BTL];
    __shared__ __attribute__((aligned(16))) float gm[4 * BT];
    __shared__ float bt[BT];
    // value-tile buffers, reused as two 64 x 64 scratch tiles by the finish
    __shared__ __attribute__((aligned(16))) float tb[2 * DK * VTL + 6 * BT * VTL];
    __shared__ float rowG[BT], rowK[BT], colP[4][BT], dbT[BT], red[8];
    float* Hs = tb;                      // h      [key][col]
    float* DHs = Hs + DK * VTL;          // dh'    [key][col]
    float* Vs = DHs + DK * VTL;          // v      [row][col]
    float* DOs = Vs + BT * VTL;          // dO
    float* DVs = DOs + BT * VTL;         // dvn
    float* Ys = DVs + BT * VTL;          // Y
    float* VNs = Ys + BT * VTL;          // v_new
    float* Zs = VNs + BT * VTL;          // Z
    float* X1 = tb;                      // finish: 64 x 64 scratch
    float* X2 = tb + BT * BTL;
    static_assert(2 * BT * BTL <= 2 * DK * VTL + 6 * BT * VTL, "scratch tiles fit the value-tile buffers");

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = blockIdx.x, head = blockIdx.y, H = a.H;
    int u, cc;
    chunk_of(a.um, ci, u, cc);
    if (u < 0) return;
    const UnitInfo ui = unit_info(a.um, u);
    const int64_t t0 = ui.start + (int64_t)cc * BT;
    int len = ui.len - cc * BT;
    len = len < 0 ? 0 : (len > BT ? BT : len);
    const int64_t ch = (int64_t)ci * H + head;
    const float lnb = a.use_exp2 ? 0.6931471805599453f : 1.0f;
    const In* vin = reinterpret_cast<const In*>(a.v);
    const In* dout = reinterpret_cast<const In*>(a.dout);

    // the value tiles of tile vt + 1 are loaded into registers while tile vt
    // is computed (28 VGPRs), and written to LDS at the next tile's top
    TileRegs<float, DK, VT> ph, pdh;
    TileRegs<In, BT, VT> pv, pdo;
    TileRegs<float, BT, VT> pdv;
    auto prefetch = [&](int vt) {
        const int vc0 = vt * VT;
        ph.issue(a.h + ch * DK * DV + vc0, DV, DK, tid);
        pdh.issue(a.dH + ch * DK * DV + vc0, DV, DK, tid);
        pv.issue(vin + (t0 * H + head) * DV + vc0, (int64_t)H * DV, len, tid);
        pdo.issue(dout + (t0 * H + head) * DV + vc0, (int64_t)H * DV, len, tid);
        pdv.issue(a.dVN + ch * BT * DV + vc0, DV, BT, tid);
    };
    load_chunk<In, false>(a, t0, ch, head, len, Ks, Qs, Ts, Ps, gm, bt, tid);
    prefetch(0);
    if (tid < BT) {
        rowG[tid] = 0.0f;
        rowK[tid] = 0.0f;
    }
    const int row0 = 16 * w;
    auto bG = [&](int row) { return gm[BT + row]; };

    // MFMA operands of this wave's rows, read once for all value tiles:
    // Tb[row0 + n][4q + G] (nonzero for 4q <= row0 + 15), Tb[4q + G][row0 + n]
    // (nonzero for 4q >= row0) and the Ks row row0 + n in 16-byte groups
    float tbr[16], tbc[16];
    f32x4 kdr[8];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int k = 4 * q + G;
        tbr[q] = Ts[(row0 + n) * BTL + k] * bt[k];
        tbc[q] = Ts[k * BTL + row0 + n] * bt[row0 + n];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) kdr[q] = *reinterpret_cast<const f32x4*>(Ks + (row0 + n) * BKL + 16 * q + 4 * G);

    f32x4 aP[4], aT[4], aQ[8], aKg[8], aKd[8];
    for (int j = 0; j < 4; ++j) { aP[j] = f32x4{0.f, 0.f, 0.f, 0.f}; aT[j] = aP[j]; }
    for (int j = 0; j < 8; ++j) { aQ[j] = f32x4{0.f, 0.f, 0.f, 0.f}; aKg[j] = aQ[j]; aKd[j] = aQ[j]; }
    float hdh = 0.0f;     // this thread's share of sum(h o dh')
    for (int vt = 0; vt < DV / VT; ++vt) {
        const int vc0 = vt * VT;
        lds_barrier();                           // the previous tile's buffers are consumed
        ph.commit(Hs, VTL, tid);
        pdh.commit(DHs, VTL, tid);
        pv.commit(Vs, VTL, tid);
        pdo.commit(DOs, VTL, tid);
        pdv.commit(DVs, VTL, tid);
        lds_barrier();
        if (vt + 1 < DV / VT) prefetch(vt + 1);
#pragma unroll
        for (int m = 0; m < DK * VT / 256; ++m) {
            const int e = tid + 256 * m, key = e / VT, cl = e - key * VT;
            hdh += Hs[key * VTL + cl] * DHs[key * VTL + cl];
        }
        // Y = V - Kd h, rows of this wave (Kd h = b^G (K h))
        {
            f32x4 kh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    kh = __builtin_amdgcn_mfma_f32_16x16x4f32(kdr[q][e], Hs[(16 * q + 4 * G + e) * VTL + n], kh, 0, 0, 0);
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + 4 * G + r;
                Ys[row * VTL + n] = Vs[row * VTL + n] - bG(row) * kh[r];
            }
        }
        lds_barrier();
        // v_new = Tb Y and Z = Tb^T dvn = dV, rows of this wave
        {
            f32x4 vn = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if (4 * q <= row0 + 15) vn = __builtin_amdgcn_mfma_f32_16x16x4f32(tbr[q], Ys[(4 * q + G) * VTL + n], vn, 0, 0, 0);
                if (4 * q >= row0) z = __builtin_amdgcn_mfma_f32_16x16x4f32(tbc[q], DVs[(4 * q + G) * VTL + n], z, 0, 0, 0);
            }
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + 4 * G + r;
                VNs[row * VTL + n] = vn[r];
                Zs[row * VTL + n] = z[r];
                if (row < len) a.dv[((t0 + row) * H + head) * DV + vc0 + n] = z[r];
            }
        }
        lds_barrier();
        // accumulate over this tile's columns (both operands column-contiguous)
        for (int j = 0; j < 4; ++j) {
            mm_rows16(aP[j], DOs + row0 * VTL, VNs + 16 * j * VTL, a.scale, G, n);
            mm_rows16(aT[j], DVs + row0 * VTL, Ys + 16 * j * VTL, 1.0f, G, n);
        }
        for (int j = 0; j < 8; ++j) {
            mm_rows16(aQ[j], DOs + row0 * VTL, Hs + 16 * j * VTL, a.scale, G, n);
            mm_rows16(aKg[j], VNs + row0 * VTL, DHs + 16 * j * VTL, 1.0f, G, n);
            mm_rows16(aKd[j], Zs + row0 * VTL, Hs + 16 * j * VTL, -1.0f, G, n);
        }
    }
    lds_barrier();

    // ---- finish. dTb (lower incl. diagonal) to X1, dP (lower incl.) to X2
    for (int j = 0; j < 4; ++j)
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + 4 * G + r, jj = 16 * j + n;
            X1[i * BTL + jj] = jj <= i ? aT[j][r] : 0.0f;
            X2[i * BTL + jj] = jj <= i ? aP[j][r] : 0.0f;
        }
    lds_barrier();
    // dbeta from Tb = T diag(beta): column sums of dTb o T
    if (tid < BT) {
        float s = 0.0f;
        for (int i = tid; i < BT; ++i) s += X1[i * BTL + tid] * Ts[i * BTL + tid];
        dbT[tid] = s;
    }
    // M1 = dT T^T with dT = dTb diag(beta), rows of this wave
    f32x4 m1[4];
    for (int j = 0; j < 4; ++j) {
        m1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        mmf<BT>(m1[j], [&](int m, int k) { return X1[(row0 + m) * BTL + k] * bt[k]; },
                [&](int k, int nn) { return Ts[(16 * j + nn) * BTL + k]; }, G, n);
    }
    lds_barrier();
    for (int j = 0; j < 4; ++j)
        for (int r = 0; r < 4; ++r) X1[(row0 + 4 * G + r) * BTL + 16 * j + n] = m1[j][r];
    lds_barrier();
    // dL = -T^T M1 (strictly lower), and G = (K K^T) o D, rows of this wave
    f32x4 dl[4], kk[4];
    for (int j = 0; j < 4; ++j) {
        dl[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        kk[j] = dl[j];
        mmf<BT>(dl[j], [&](int m, int k) { return Ts[k * BTL + row0 + m]; },
                [&](int k, int nn) { return X1[k * BTL + 16 * j + nn]; }, G, n);
        mmf<DK>(kk[j], [&](int m, int k) { return Ks[(row0 + m) * BKL + k]; },
                [&](int k, int nn) { return Ks[(16 * j + nn) * BKL + k]; }, G, n);
    }
    lds_barrier();
    // element terms of L and P: dbeta_i += sum_j dL_ij G_ij, dG = beta_i dL,
    // the G_i / G_j parts of the gate gradient, and dG o D, dP o D in place
    float rb[4] = {0.f, 0.f, 0.f, 0.f}, rg[4] = {0.f, 0.f, 0.f, 0.f}, cg[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < 4; ++j)
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + 4 * G + r, jj = 16 * j + n;
            const float d = jj <= i ? fpow(gm[i] - gm[jj], a.use_exp2) : 0.0f;
            const float lij = jj < i ? -dl[j][r] : 0.0f;              // dL
            const float gij = kk[j][r] * d;                           // (k_i . k_j) D_ij
            const float dgg = bt[i] * lij;                            // dG
            const float pij = Ps[i * BTL + jj], dpij = X2[i * BTL + jj];
            rb[r] += lij * gij;
            const float t = lnb * (dgg * gij + dpij * pij);
            rg[r] += t;
            cg[j] -= t;
            X1[i * BTL + jj] = dgg * d;
            X2[i * BTL + jj] = dpij * d;
        }
    // column sums over this wave's rows (lanes 16 apart), one partial per
    // wave, added in a fixed order below: no float atomics, so the result
    // is the same on every run
    for (int j = 0; j < 4; ++j) {
        cg[j] += __shfl_xor(cg[j], 16, 64);
        cg[j] += __shfl_xor(cg[j], 32, 64);
    }
    if (G == 0)
        for (int j = 0; j < 4; ++j) colP[w][16 * j + n] = cg[j];
    // row sums over the 16 lanes of each group
    for (int r = 0; r < 4; ++r)
        for (int s = 1; s < 16; s <<= 1) {
            rb[r] += __shfl_xor(rb[r], s, 16);
            rg[r] += __shfl_xor(rg[r], s, 16);
        }
    if (n == 0)
        for (int r = 0; r < 4; ++r) {
            atomicAdd(&rowG[row0 + 4 * G + r], rg[r]);
            atomicAdd(&dbT[row0 + 4 * G + r], rb[r]);
        }
    lds_barrier();
    // dq, dk, rows of this wave: the products with dG o D and dP o D, then
    // b^G dQd, b^G dKd + b^{G_L - G} dKg, and their gate terms
    float rq[4] = {0.f, 0.f, 0.f, 0.f}, rk[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < 8; ++j) {
        f32x4 q1 = {0.f, 0.f, 0.f, 0.f}, k1 = q1;
        mmf<BT>(q1, [&](int m, int k) { return X2[(row0 + m) * BTL + k]; },
                [&](int k, int nn) { return Ks[k * BKL + 16 * j + nn]; }, G, n);
        mmf<BT>(k1, [&](int m, int k) { return X1[(row0 + m) * BTL + k]; },
                [&](int k, int nn) { return Ks[k * BKL + 16 * j + nn]; }, G, n);
        mmf<BT>(k1, [&](int m, int k) { return X1[k * BTL + row0 + m]; },
                [&](int k, int nn) { return Ks[k * BKL + 16 * j + nn]; }, G, n);
        mmf<BT>(k1, [&](int m, int k) { return X2[k * BTL + row0 + m]; },
                [&](int k, int nn) { return Qs[k * BKL + 16 * j + nn]; }, G, n);
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + 4 * G + r, d = 16 * j + n;
            const float bg = gm[BT + i], blg = gm[2 * BT + i];
            const float qv = Qs[i * BKL + d], kv = Ks[i * BKL + d];
            const float dqv = q1[r] + bg * aQ[j][r];
            const float dkv = k1[r] + bg * aKd[j][r] + blg * aKg[j][r];
            // the Kg term (ln b dKg Kg) goes to dg as a prefix over earlier
            // rows: its - part here and its + part in G_L's gradient cancel
            // for every row from i on
            rq[r] += lnb * (aQ[j][r] * bg * qv + aKd[j][r] * bg * kv);
            rk[r] += lnb * aKg[j][r] * blg * kv;
            if (i < len) {
                a.dq[((t0 + i) * H + head) * DK + d] = dqv;
                a.dk[((t0 + i) * H + head) * DK + d] = dkv;
            }
        }
    }
    for (int r = 0; r < 4; ++r)
        for (int s = 1; s < 16; s <<= 1) {
            rq[r] += __shfl_xor(rq[r], s, 16);
            rk[r] += __shfl_xor(rk[r], s, 16);
        }
    if (n == 0)
        for (int r = 0; r < 4; ++r) {
            atomicAdd(&rowG[row0 + 4 * G + r], rq[r]);
            rowK[row0 + 4 * G + r] = rk[r];
        }
    // the state decay's term of G_L: lnb gamma sum(h o dh'), over the workgroup
    float tl = lnb * gm[3 * BT] * hdh;
    for (int s = 1; s < 64; s <<= 1) tl += __shfl_xor(tl, s, 64);
    if (lane == 0) red[w] = tl;
    lds_barrier();
    // dg: reverse cumulative sum over the chunk's rows of the gate gradient,
    // with the state decay's term entering at the last valid row, plus the
    // exclusive prefix of the Kg terms
    if (w == 0) {
        const float gl = red[0] + red[1] + red[2] + red[3];
        const float colG = ((colP[0][lane] + colP[1][lane]) + colP[2][lane]) + colP[3][lane];
        float x = lane < len ? rowG[lane] + colG + (lane == len - 1 ? gl : 0.0f) : 0.0f;
        const float kg = lane < len ? rowK[lane] : 0.0f;
        float y = kg;
        for (int s = 1; s < 64; s <<= 1) {
            const float xd = __shfl_down(x, s, 64), yu = __shfl_up(y, s, 64);
            if (lane + s < 64) x += xd;
            if (lane >= s) y += yu;
        }
        x += y - kg;
        if (lane < len) {
            a.dg[(t0 + lane) * H + head] = x;
            a.dbeta[(t0 + lane) * H + head] = dbT[lane];
        }
    }
}

// Per-key per-chunk gradients at eight waves, two per SIMD. Waves w and
// w + 4 share token rows 16w .. +15: group 0 (waves 0..3) forms Y and v_new
// and accumulates dP, group 1 forms dvn and Z (= dV) and accumulates dTb,
// and each accumulates dQd, dKg and dKd for key tiles 2jj + group (jj =
// 0..3), the tiles its waves take in the finish. Waves 0..3 stage the value
// tiles.
template <class In>
__global__ __launch_bounds__(512, 1) void bwd_grad_kernel_pk(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) float Ks[BT * BKL];
    __shared__ __attribute__((aligned(16))) float Qs[BT * BKL];
    __shared__ __attribute__((aligned(16))) float Ts[BT * BTL];     // T
    __shared__ __attribute__((aligned(16))) float Ps[BT * BTL];
    __shared__ float bt[BT];
    // value-tile buffers, reused as two 64 x 64 scratch tiles by the finish
    __shared__ __attribute__((aligned(16))) float tb[2 * DK * VTL + 6 * BT * VTL];
    __shared__ float dbT[BT], brs[2 * BT];
    float* Hs = tb;                      // h      [key][col]
    float* DHs = Hs + DK * VTL;          // dh'    [key][col]
    float* Vs = DHs + DK * VTL;          // v      [row][col]
    float* DOs = Vs + BT * VTL;          // dO
    float* DVs = DOs + BT * VTL;         // dvn
    float* Ys = DVs + BT * VTL;          // Y
    float* VNs = Ys + BT * VTL;          // v_new
    float* Zs = VNs + BT * VTL;          // Z
    float* X1 = tb;                      // finish: 64 x 64 scratch
    float* X2 = tb + BT * BTL;

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6), w = w8 & 3, grp = w8 >> 2;
    const bool ld = tid < 256;                   // the threads that stage tiles
    const int ci = blockIdx.x, head = blockIdx.y, H = a.H;
    int u, cc;
    chunk_of(a.um, ci, u, cc);
    if (u < 0) return;
    const UnitInfo ui = unit_info(a.um, u);
    const int64_t t0 = ui.start + (int64_t)cc * BT;
    int len = ui.len - cc * BT;
    len = len < 0 ? 0 : (len > BT ? BT : len);
    const int64_t ch = (int64_t)ci * H + head;
    const In* vin = reinterpret_cast<const In*>(a.v);
    const In* dout = reinterpret_cast<const In*>(a.dout);

    TileRegs<float, DK, VT> ph, pdh;
    TileRegs<In, BT, VT> pv, pdo;
    auto prefetch = [&](int vt) {
        if (!ld) return;
        const int vc0 = vt * VT;
        ph.issue(a.h + ch * DK * DV + vc0, DV, DK, tid);
        pdh.issue(a.dH + ch * DK * DV + vc0, DV, DK, tid);
        pv.issue(vin + (t0 * H + head) * DV + vc0, (int64_t)H * DV, len, tid);
        pdo.issue(dout + (t0 * H + head) * DV + vc0, (int64_t)H * DV, len, tid);
    };
    {
        // k b^G (for Y) in Ks, T, k b^{G_L - G} (for dvn) in Qs and P, all
        // four loads in flight together; q, k and G come in key slices in
        // the finish
        TileRegs<float, BT, DK> rkd, rkg;
        TileRegs<float, BT, BT> rt, rp;
        prefetch(0);
        if (ld) {
            rkd.issue(reinterpret_cast<const float*>(a.ws.kd) + ch * (BT * DK), DK, BT, tid);
            rt.issue(reinterpret_cast<const float*>(a.ws.Tm) + ch * (BT * BT), BT, BT, tid);
            rkg.issue(reinterpret_cast<const float*>(a.ws.kg) + ch * (BT * DK), DK, BT, tid);
            rp.issue(reinterpret_cast<const float*>(a.ws.P) + ch * (BT * BT), BT, BT, tid);
        }
        if (tid < BT) bt[tid] = tid < len ? ldf(reinterpret_cast<const In*>(a.beta), (t0 + tid) * H + head) : 0.0f;
        if (ld) {
            rkd.commit(Ks, BKL, tid);
            rt.commit(Ts, BTL, tid);
            rkg.commit(Qs, BKL, tid);
            rp.commit(Ps, BTL, tid);
        }
        lds_barrier();
    }
    const int row0 = 16 * w;

    // MFMA operands of this wave's rows, read once for all value tiles.
    // Group 0: Tb[row0 + n][4q + G] (nonzero for 4q <= row0 + 15) and the Kd
    // row; group 1: Tb[4q + G][row0 + n] and P[4q + G][row0 + n] (nonzero for
    // 4q >= row0) and the Kg row.
    float t1[16], pc[16];
    f32x4 kx[8];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int k = 4 * q + G;
        t1[q] = grp == 0 ? Ts[(row0 + n) * BTL + k] * bt[k] : Ts[k * BTL + row0 + n] * bt[row0 + n];
        pc[q] = grp == 0 ? 0.0f : Ps[k * BTL + row0 + n];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
        kx[q] = *reinterpret_cast<const f32x4*>((grp == 0 ? Ks : Qs) + (row0 + n) * BKL + 16 * q + 4 * G);

    f32x4 aPT[4], aQ[4], aKg[4], aKd[4];         // dP (group 0) or dTb (group 1); key tiles 2jj + grp
    for (int j = 0; j < 4; ++j) {
        aPT[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        aQ[j] = aPT[j];
        aKg[j] = aPT[j];
        aKd[j] = aPT[j];
    }
    float hk[4] = {0.f, 0.f, 0.f, 0.f};         // per key: keys (tid >> 4) + 32m, column tid & 15
    for (int vt = 0; vt < DV / VT; ++vt) {
        const int vc0 = vt * VT;
        lds_barrier();                           // the previous tile's buffers are consumed
        if (ld) {
            ph.commit(Hs, VTL, tid);
            pdh.commit(DHs, VTL, tid);
            pv.commit(Vs, VTL, tid);
            pdo.commit(DOs, VTL, tid);
        }
        lds_barrier();
        if (vt + 1 < DV / VT) prefetch(vt + 1);
#pragma unroll
        for (int m = 0; m < DK * VT / 512; ++m) {
            const int e = tid + 512 * m, key = e / VT, cl = e - key * VT;
            hk[m] += Hs[key * VTL + cl] * DHs[key * VTL + cl];
        }
        if (grp == 0) {
            // Y = V - Kd h, rows of this wave
            f32x4 kh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    kh = __builtin_amdgcn_mfma_f32_16x16x4f32(kx[q][e], Hs[(16 * q + 4 * G + e) * VTL + n], kh, 0, 0, 0);
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + 4 * G + r;
                Ys[row * VTL + n] = Vs[row * VTL + n] - kh[r];
            }
        } else {
            // dvn = Kg dh' + scale P^T dO, rows of this wave (P[j][i] = 0 for j < i)
            f32x4 kd = {0.f, 0.f, 0.f, 0.f}, pd = kd;
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    kd = __builtin_amdgcn_mfma_f32_16x16x4f32(kx[q][e], DHs[(16 * q + 4 * G + e) * VTL + n], kd, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (4 * q >= row0)
                    pd = __builtin_amdgcn_mfma_f32_16x16x4f32(pc[q], DOs[(4 * q + G) * VTL + n], pd, 0, 0, 0);
            for (int r = 0; r < 4; ++r) DVs[(row0 + 4 * G + r) * VTL + n] = kd[r] + a.scale * pd[r];
        }
        lds_barrier();
        if (grp == 0) {
            // v_new = Tb Y, rows of this wave
            f32x4 vn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (4 * q <= row0 + 15) vn = __builtin_amdgcn_mfma_f32_16x16x4f32(t1[q], Ys[(4 * q + G) * VTL + n], vn, 0, 0, 0);
            for (int r = 0; r < 4; ++r) VNs[(row0 + 4 * G + r) * VTL + n] = vn[r];
        } else {
            // Z = Tb^T dvn = dV, rows of this wave
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (4 * q >= row0) z = __builtin_amdgcn_mfma_f32_16x16x4f32(t1[q], DVs[(4 * q + G) * VTL + n], z, 0, 0, 0);
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + 4 * G + r;
                Zs[row * VTL + n] = z[r];
                if (row < len) a.dv[((t0 + row) * H + head) * DV + vc0 + n] = z[r];
            }
        }
        lds_barrier();
        // accumulate over this tile's columns (both operands column-contiguous)
        for (int j = 0; j < 4; ++j) {
            if (grp == 0) mm_rows16(aPT[j], DOs + row0 * VTL, VNs + 16 * j * VTL, a.scale, G, n);
            else mm_rows16(aPT[j], DVs + row0 * VTL, Ys + 16 * j * VTL, 1.0f, G, n);
        }
        for (int jj = 0; jj < 4; ++jj) {
            const int j = 2 * jj + grp;
            mm_rows16(aQ[jj], DOs + row0 * VTL, Hs + 16 * j * VTL, a.scale, G, n);
            mm_rows16(aKg[jj], VNs + row0 * VTL, DHs + 16 * j * VTL, 1.0f, G, n);
            mm_rows16(aKd[jj], Zs + row0 * VTL, Hs + 16 * j * VTL, -1.0f, G, n);
        }
    }
    lds_barrier();

    // ---- finish. dTb (group 1) to X1, dP (group 0) to X2, lower incl. diagonal
    {
        float* X = grp == 0 ? X2 : X1;
        for (int j = 0; j < 4; ++j)
            for (int r = 0; r < 4; ++r) {
                const int i = row0 + 4 * G + r, jj = 16 * j + n;
                X[i * BTL + jj] = jj <= i ? aPT[j][r] : 0.0f;
            }
    }
    lds_barrier();
    // dbeta from Tb = T diag(beta): column sums of dTb o T
    if (tid < BT) {
        float sc = 0.0f;
        for (int i = tid; i < BT; ++i) sc += X1[i * BTL + tid] * Ts[i * BTL + tid];
        dbT[tid] = sc;
    }
    // M1 = dT T^T with dT = dTb diag(beta), rows of this wave, column blocks 2 grp, 2 grp + 1
    f32x4 m1[2];
    for (int jh = 0; jh < 2; ++jh) {
        const int j = 2 * grp + jh;
        m1[jh] = f32x4{0.f, 0.f, 0.f, 0.f};
        mmf<BT>(m1[jh], [&](int m, int k) { return X1[(row0 + m) * BTL + k] * bt[k]; },
                [&](int k, int nn) { return Ts[(16 * j + nn) * BTL + k]; }, G, n);
    }
    lds_barrier();
    for (int jh = 0; jh < 2; ++jh)
        for (int r = 0; r < 4; ++r) X1[(row0 + 4 * G + r) * BTL + 16 * (2 * grp + jh) + n] = m1[jh][r];
    lds_barrier();
    // dL = -T^T M1 (strictly lower), rows of this wave, the same column blocks
    f32x4 dl[2];
    for (int jh = 0; jh < 2; ++jh) {
        const int j = 2 * grp + jh;
        dl[jh] = f32x4{0.f, 0.f, 0.f, 0.f};
        mmf<BT>(dl[jh], [&](int m, int k) { return Ts[k * BTL + row0 + m]; },
                [&](int k, int nn) { return X1[k * BTL + 16 * j + nn]; }, G, n);
    }
    lds_barrier();
    finish_per_key8<In>(a, t0, head, len, row0, w, w8, grp, G, n, lane, tid, dl, aQ, aKd, aKg, hk, X1, X2, Ks, Qs,
                        bt, dbT, brs);
}

// ------------------------------------------------------------------ reverse state pass, per-key gate
// The per-key reverse chunk step as an affine map of the state gradient, in
// fp32 (D = dL/dh at the chunk's exit, D' at its entry):
//   D' = A D + scale U^T dO,  A = diag(b^{G_L}) - W^T Kg,  U = Qd - P W,  W = Tb Kd
// with Kd, Kg, Qd the prepared gated tiles (k b^G, k b^{G_L - G}, q b^G):
// the per-key gamma, Qd^T dO and Kd^T Tb^T (Kg D + scale P^T dO) of the
// three-phase step regrouped. bwd_transfer_kernel_pk forms A and U of every
// chunk at once, and bwd_dh_kernel_pkr runs the sequential pass with one load
// phase per chunk (the next chunk's A, U and dO prefetched into registers);
// the per-chunk gradient kernel forms dvn = Kg D + scale P^T dO itself.

// One workgroup of four waves per (chunk, head), two per compute unit: wave w
// forms rows 16w .. +15 of W, rows 32w .. +31 of A and rows 16w .. +15 of U.
// Kd, then Kg, and W sit transposed in LDS ([key][row]), so that every
// product reads both operands along its contraction with 16-byte loads; the
// wave's own rows of T and P (lower triangular: only the first w + 1 16-wide
// column blocks are nonzero) go straight from memory into MFMA operand
// registers. The next tile's loads are in flight while the current product
// runs. A comes out of a transposed product, so a lane holds four consecutive
// columns of one row (16-byte stores). U^T ([key][row]) overwrites the
// chunk-head's Qd tile, which nothing reads after this kernel.
constexpr int KTL = BT + 4;     // row stride (floats) of the transposed 128 x 64 tiles

// a 64 x 128 fp32 tile in registers, 16 x 16 blocks per wave and load, for a
// transposed store into LDS in which the 64 lanes of a store hit 64 banks
struct TileT {
    f32x4 v[8];
    __device__ __forceinline__ void issue(const float* src, int w, int l) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int bi = 4 * i + w, r = 16 * (bi & 3) + (l & 15), c = 16 * (bi >> 2) + 4 * (l >> 4);
            v[i] = *reinterpret_cast<const f32x4*>(src + r * DK + c);
        }
    }
    __device__ __forceinline__ void commit(float* dst, int w, int l) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int bi = 4 * i + w, r = 16 * (bi & 3) + (l & 15), c = 16 * (bi >> 2) + 4 * (l >> 4);
            for (int j = 0; j < 4; ++j) dst[(c + j) * KTL + r] = v[i][j];
        }
    }
};

template <class In>
__global__ __launch_bounds__(256, 2) void bwd_transfer_kernel_pk(BwdArgs a, float* Aw) {
    __shared__ __attribute__((aligned(16))) float Xt[DK * KTL];   // Kd^T, then Kg^T
    __shared__ __attribute__((aligned(16))) float Wt[DK * KTL];   // W^T
    __shared__ float bt[BT], gl[DK];

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = blockIdx.x, head = blockIdx.y, H = a.H;
    int u, cc;
    chunk_of(a.um, ci, u, cc);
    if (u < 0) return;
    const UnitInfo ui = unit_info(a.um, u);
    const int64_t t0 = ui.start + (int64_t)cc * BT;
    int len = ui.len - cc * BT;
    len = len < 0 ? 0 : (len > BT ? BT : len);
    const int64_t ch = (int64_t)ci * H + head;
    const int row0 = 16 * w;
    float* qg = reinterpret_cast<float*>(a.ws.qg) + ch * (BT * DK);
    const float* Tm = reinterpret_cast<const float*>(a.ws.Tm) + ch * (BT * BT) + (row0 + n) * BT + 4 * G;
    const float* Pm = reinterpret_cast<const float*>(a.ws.P) + ch * (BT * BT) + (row0 + n) * BT + 4 * G;

    TileT tx;                                    // Kd, then Kg
    tx.issue(reinterpret_cast<const float*>(a.ws.kd) + ch * (BT * DK), w, lane);
    f32x4 tf[4], pf[4];                          // T, P: row row0 + n, columns 16 kk + 4G .. +3
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        tf[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (kk <= w) tf[kk] = *reinterpret_cast<const f32x4*>(Tm + 16 * kk);
    }
    if (tid < BT) bt[tid] = tid < len ? ldf(reinterpret_cast<const In*>(a.beta), (t0 + tid) * H + head) : 0.0f;
    if (tid < DK) gl[tid] = fpow(a.ws.gamL[ch * DK + tid], a.use_exp2);
    tx.commit(Xt, w, lane);                      // Kd^T
    lds_barrier();
    tx.issue(reinterpret_cast<const float*>(a.ws.kg) + ch * (BT * DK), w, lane);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        pf[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (kk <= w) pf[kk] = *reinterpret_cast<const f32x4*>(Pm + 16 * kk);
        for (int e = 0; e < 4; ++e) tf[kk][e] *= bt[16 * kk + 4 * G + e];   // T diag(beta)
    }
    // W = Tb Kd, rows of this wave, stored as W^T
    for (int ct = 0; ct < DK / 16; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk > w) continue;
            const f32x4 y = *reinterpret_cast<const f32x4*>(Xt + (16 * ct + n) * KTL + 16 * kk + 4 * G);
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tf[kk][e], y[e], acc, 0, 0, 0);
        }
        *reinterpret_cast<f32x4*>(&Wt[(16 * ct + n) * KTL + row0 + 4 * G]) = acc;
    }
    lds_barrier();
    tx.commit(Xt, w, lane);                      // Kg^T
    f32x4 qd[DK / 16];                           // Qd[row0 + 4G + r][16 ct + n]
#pragma unroll
    for (int ct = 0; ct < DK / 16; ++ct)
        for (int r = 0; r < 4; ++r) qd[ct][r] = qg[(row0 + 4 * G + r) * DK + 16 * ct + n];
    lds_barrier();
    // A = diag(b^{G_L}) - W^T Kg, rows 32w .. 32w+31: lane holds A[k1 + n][16 ct + 4G .. +3]
    float* Ac = Aw + ch * (DK * DK);
    for (int rt = 0; rt < 2; ++rt) {
        const int k1 = 32 * w + 16 * rt;
        for (int ct = 0; ct < DK / 16; ++ct) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mm_rowsk<BT>(acc, Xt + 16 * ct * KTL, KTL, Wt + k1 * KTL, KTL, G, n);
            f32x4 o;
            for (int r = 0; r < 4; ++r) o[r] = (k1 + n == 16 * ct + 4 * G + r ? gl[k1 + n] : 0.0f) - acc[r];
            *reinterpret_cast<f32x4*>(Ac + (k1 + n) * DK + 16 * ct + 4 * G) = o;
        }
    }
    // U = Qd - P W, rows of this wave: lane holds U[row0 + 4G + r][16 ct + n]
    f32x4 uo[DK / 16];
    for (int ct = 0; ct < DK / 16; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk > w) continue;
            const f32x4 y = *reinterpret_cast<const f32x4*>(Wt + (16 * ct + n) * KTL + 16 * kk + 4 * G);
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pf[kk][e], y[e], acc, 0, 0, 0);
        }
        uo[ct] = qd[ct] - acc;
    }
    // U^T ([key][row]) over the tile: every wave has read its Qd rows
    __syncthreads();
    for (int ct = 0; ct < DK / 16; ++ct)
        *reinterpret_cast<f32x4*>(qg + (16 * ct + n) * BT + row0 + 4 * G) = uo[ct];
}

// The sequential pass: one workgroup of eight waves per (unit, head, 16 NCT
// value columns), one per compute unit (two waves per SIMD); wave w keeps D
// for keys 16w .. 16w+15 in fp32 registers and a copy in LDS as
// [column][key]. Its rows of A and of U^T come straight from memory into
// MFMA operand registers, one chunk ahead (two register sets, taken in
// turn); dO goes through LDS as [column][row]. D and dO are double-buffered
// in LDS, so one barrier per chunk hands both over. dh' of every chunk goes
// to the workspace.
constexpr int DTL = BT + 4;     // row stride (floats) of the transposed dO tile
constexpr int PKR = 512;        // threads of the per-key sequential pass

template <class In, int NCT>
__global__ __launch_bounds__(PKR, 1) void bwd_dh_kernel_pkr(BwdArgs a, const float* Aw) {
    constexpr int NC = 16 * NCT;
    __shared__ __attribute__((aligned(16))) float dhT[2][NC * BKL];  // D [column][key]
    __shared__ __attribute__((aligned(16))) float dOT[2][NC * DTL];  // dO [column][row]

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int tile = slot % (DV / NC), pair = (slot / (DV / NC)) * 8 + xcd;
    if (pair >= a.n_pairs) return;
    const int u = pair / H, head = pair - u * H;
    const UnitInfo ui = uniform(unit_info(a.um, u));
    const int c0 = tile * NC;
    const int64_t uh = (int64_t)u * H + head;
    const float* Uw = reinterpret_cast<const float*>(a.ws.qg);
    const int key0 = 16 * w;
    const bool ld = tid < 256;                   // the threads that stage dO

    f32x4 dh[NCT];
    const int b_last = (ui.nch - 1) & 1;
    for (int ct = 0; ct < NCT; ++ct) {
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + 4 * G + r, col = 16 * ct + n;
            dh[ct][r] = a.dht ? a.dht[(uh * DK + key) * DV + c0 + col] : 0.0f;
        }
        *reinterpret_cast<f32x4*>(&dhT[b_last][(16 * ct + n) * BKL + key0 + 4 * G]) = dh[ct];
    }

    // operand registers: A[key0 + n][16kb + 4G .. +3], U^T[key0 + n][16rb + 4G .. +3]
    f32x4 A0[8], U0[4], A1[8], U1[4];
    TileRegs<In, BT, NC> pd;
    auto issue = [&](int cc, f32x4 (&Ar)[8], f32x4 (&Ur)[4]) {
        int l = ui.len - cc * BT;
        l = l > BT ? BT : l;
        const int64_t tt = ui.start + (int64_t)cc * BT, chh = (int64_t)(ui.cbase + cc) * H + head;
        const float* ap = Aw + chh * (DK * DK) + (key0 + n) * DK + 4 * G;
        const float* up = Uw + chh * (DK * BT) + (key0 + n) * BT + 4 * G;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) Ar[kb] = *reinterpret_cast<const f32x4*>(ap + 16 * kb);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) Ur[rb] = *reinterpret_cast<const f32x4*>(up + 16 * rb);
        if (ld) pd.issue(reinterpret_cast<const In*>(a.dout) + (tt * H + head) * DV + c0, (int64_t)H * DV, l, tid);
    };
    auto step = [&](int c, const f32x4 (&Ar)[8], const f32x4 (&Ur)[4], f32x4 (&An)[8], f32x4 (&Un)[4]) {
        const int64_t ch = (int64_t)(ui.cbase + c) * H + head;
        const int b = c & 1;
        if (ld) pd.commit_tr(dOT[b], DTL, tid);
        if (c > 0) issue(c - 1, An, Un);
        for (int ct = 0; ct < NCT; ++ct)
            for (int r = 0; r < 4; ++r) a.dH[(ch * DK + key0 + 4 * G + r) * DV + c0 + 16 * ct + n] = dh[ct][r];
        lds_barrier();                           // D and dO of this chunk are in LDS
        // D' = A D + scale U^T dO, keys key0 .. +15
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 ad = {0.f, 0.f, 0.f, 0.f}, ae = ad;
            const float* dcol = dhT[b] + (16 * ct + n) * BKL + 4 * G;
            const float* ocol = dOT[b] + (16 * ct + n) * DTL + 4 * G;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const f32x4 y = *reinterpret_cast<const f32x4*>(dcol + 16 * kb);
#pragma unroll
                for (int e = 0; e < 4; ++e) ad = __builtin_amdgcn_mfma_f32_16x16x4f32(Ar[kb][e], y[e], ad, 0, 0, 0);
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const f32x4 y = *reinterpret_cast<const f32x4*>(ocol + 16 * rb);
#pragma unroll
                for (int e = 0; e < 4; ++e) ae = __builtin_amdgcn_mfma_f32_16x16x4f32(Ur[rb][e], y[e], ae, 0, 0, 0);
            }
            for (int r = 0; r < 4; ++r) dh[ct][r] = ad[r] + a.scale * ae[r];
            *reinterpret_cast<f32x4*>(&dhT[b ^ 1][(16 * ct + n) * BKL + key0 + 4 * G]) = dh[ct];
        }
    };
    if (ui.nch > 0) issue(ui.nch - 1, A0, U0);
    for (int c = ui.nch - 1; c >= 0; c -= 2) {
        step(c, A0, U0, A1, U1);
        if (c >= 1) step(c - 1, A1, U1, A0, U0);
    }
    if (a.dh0)
        for (int ct = 0; ct < NCT; ++ct)
            for (int r = 0; r < 4; ++r) a.dh0[(uh * DK + key0 + 4 * G + r) * DV + c0 + 16 * ct + n] = dh[ct][r];
}

// ------------------------------------------------------------------ per-chunk gradients, bf16 inputs, scalar gate
// The same gradients as bwd_grad_kernel, with every tile in LDS as fp16 (the
// bf16 inputs exactly, the fp32 states, T, P and intermediates rounded once)
// and every product on the fp16 16x16x32 MFMA with fp32 accumulation.
// Operand fragments: lane (G, n) holds the 8 values of k-slots 8G .. 8G+7 (A:
// of row n; B: of column n). frag_row reads them from a tile whose rows run
// along k (one 16-byte read); frag_col from a tile whose columns run along k
// (two transposed 8-byte reads). Products whose result stays in registers or
// goes to LDS are formed transposed, with the wave's 16 token rows as the
// MFMA's n index: lane (G, n) then holds row 16w + n at the 4 consecutive
// columns 4G .. 4G+3 of each 16-column block, stored with one 8-byte (fp16)
// or 16-byte (fp32) write. Blocks that the triangular structure makes zero
// (T, Tb, P, dTb, dP and dL are triangular) are skipped per wave.
constexpr int HK = DK + 8;      // row stride (halves) of the 64 x 128 k and q tiles
constexpr int HT = BT + 8;      // row stride of the 64 x 64 tiles
constexpr int BTL4 = BT + 4;    // row stride (floats) of a 64 x 64 fp32 tile read 16 bytes at a time
constexpr int HVT = 32;         // value columns per tile
constexpr int HV = HVT + 8;     // row stride of the value tiles

__device__ __forceinline__ f16x8 frag_row(const f16* t, int ld, int row, int k0, int G) {
    return *reinterpret_cast<const f16x8*>(t + row * ld + k0 + 8 * G);
}
// lane (G, n): t[k0 + 8G + e][col0 + n], e = 0..7. In a 16-lane group the
// transposed read hands lane n column n of the 4 rows that lanes 4e .. 4e+3
// address (each 4 consecutive values of row e).
__device__ __forceinline__ f16x8 frag_col(const f16* t, int ld, int k0, int col0, int G, int n) {
    const f16* p = t + (k0 + 8 * G + (n >> 2)) * ld + col0 + 4 * (n & 3);
    const f16x4 x = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p)));
    const f16x4 y = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p + 4 * ld)));
    f16x8 f;
    for (int e = 0; e < 4; ++e) {
        f[e] = x[e];
        f[e + 4] = y[e];
    }
    return f;
}
__device__ __forceinline__ void mma_h(f32x4& c, f16x8 a, f16x8 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void st4h(f16* p, f32x4 x) {
    f16x4 h;
    for (int e = 0; e < 4; ++e) h[e] = (f16)x[e];
    *reinterpret_cast<f16x4*>(p) = h;
}
// Cross-lane sums without LDS traffic. row_sum16: 16 per-lane values summed
// over the 16 lanes of each row by recursive halving (partners 8, 4, 2, 1
// apart: row_ror:8, swizzle xor 4, quad_perm), so that lane n ends with the
// row's total of value n. pair16 / pair32: a value summed with that of the
// lane 16 / 32 apart (v_permlane16_swap / v_permlane32_swap of the value
// with itself); both together give the sum over the four rows.
template <int CTRL>
__device__ __forceinline__ float dpp_h(float x) {
    return u2f(__builtin_amdgcn_update_dpp(0u, f2u(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16(float (&v)[16], int n) {
    const bool up8 = n & 8, up4 = n & 4, up2 = n & 2, up1 = n & 1;
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = (up8 ? v[8 + m] : v[m]) + dpp_h<0x128>(up8 ? v[m] : v[8 + m]);
#pragma unroll
    for (int m = 0; m < 4; ++m)
        v[m] = (up4 ? v[4 + m] : v[m]) + u2f(__builtin_amdgcn_ds_swizzle((int)f2u(up4 ? v[m] : v[4 + m]), 0x101f));
#pragma unroll
    for (int m = 0; m < 2; ++m) v[m] = (up2 ? v[2 + m] : v[m]) + dpp_h<0x4e>(up2 ? v[m] : v[2 + m]);
    return (up1 ? v[1] : v[0]) + dpp_h<0xb1>(up1 ? v[0] : v[1]);
}
__device__ __forceinline__ float pair16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    return u2f(r[0]) + u2f(r[1]);
}
__device__ __forceinline__ float pair32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return u2f(r[0]) + u2f(r[1]);
}
__device__ __forceinline__ f32x4 ld4h(const f16* p) {
    const f16x4 h = *reinterpret_cast<const f16x4*>(p);
    return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}

// ------------------------------------------------------------------ reverse state pass, bf16 inputs, scalar gate
// Regrouped, the reverse chunk step is an affine map of the state gradient
// (D = dL/dh at the chunk's exit, D' at its entry):
//   D' = gamma D + scale Qd^T dO - Kd^T Z,  Z = Tb^T dvn,  dvn = Kg D + scale P^T dO
//      = A D + scale U^T dO,   A = gamma I - W^T Kg,  U = Qd - P W,  W = Tb Kd
// (W is the WY form's w; A is the transpose of the chunk's transfer map of
// the forward, h' = A^T h + ...). A and U depend on the chunk only, so
// bwd_transfer_kernel_h forms them for every chunk at once, and the
// sequential pass is one 128 x 128 product and one barrier per chunk.

// A (128 x 128, [key'][key]) and U (64 x 128, [row][key]) of every chunk-head,
// fp16: one workgroup of four waves per (chunk, head). W = T diag(beta b^G) K
// first (wave w: rows 16w .. +15), then A (wave w: rows 32w .. +31) and U
// (rows 16w .. +15), formed transposed so that each lane holds 4 consecutive
// columns of one row.
__global__ __launch_bounds__(256) void bwd_transfer_kernel_h(BwdArgs a, f16* Aw, f16* Uw) {
    __shared__ __attribute__((aligned(16))) f16 Kh[BT * HK];     // K
    __shared__ __attribute__((aligned(16))) f16 Kgh[BT * HK];    // Kg = diag(b^{G_L - G}) K
    __shared__ __attribute__((aligned(16))) f16 Tgh[BT * HT];    // T diag(beta b^G)
    __shared__ __attribute__((aligned(16))) f16 Ph[BT * HT];
    __shared__ __attribute__((aligned(16))) f16 Wh[BT * HK];     // W
    __shared__ __attribute__((aligned(16))) float gm[4 * BT];    // G, b^G, b^{G_L - G}, b^{G_L}

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = blockIdx.x, head = blockIdx.y, H = a.H;
    int u, cc;
    chunk_of(a.um, ci, u, cc);
    if (u < 0) return;
    const UnitInfo ui = unit_info(a.um, u);
    const int64_t t0 = ui.start + (int64_t)cc * BT;
    int len = ui.len - cc * BT;
    len = len < 0 ? 0 : (len > BT ? BT : len);
    const int64_t ch = (int64_t)ci * H + head;
    const bf16* bin = reinterpret_cast<const bf16*>(a.beta);
    const int row0 = 16 * w, im = row0 + n;
    const int lo_js = w >= 2 ? 2 : 1;            // 32-row steps i <= j can reach
    const float* gam = a.ws.gam + ch * (GAMR * BT);
    // q of this lane's row im for U, loaded with the tiles (rows past the
    // chunk end: zero)
    u32x2 qv[8];
    {
        const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + ((t0 + (im < len ? im : 0)) * H + head) * DK;
        for (int kb = 0; kb < 8; ++kb)
            qv[kb] = im < len ? *reinterpret_cast<const u32x2*>(qrow + 16 * kb + 4 * G) : u32x2{0u, 0u};
    }
    {
        TileRegs<bf16, BT, DK> tk;
        TileRegs<f16, BT, BT> tt, tp;
        tk.issue(reinterpret_cast<const bf16*>(a.k) + (t0 * H + head) * DK, (int64_t)H * DK, len, tid);
        tt.issue(reinterpret_cast<const f16*>(a.ws.Tm) + ch * (BT * BT), BT, BT, tid);
        tp.issue(reinterpret_cast<const f16*>(a.ws.P) + ch * (BT * BT), BT, BT, tid);
        // beta (raw, past the chunk end zero) and b^G of this thread's T
        // columns 8 (tid & 7) + j; b^{G_L - G} of its k rows 16 i + tid / 16
        const rsrc_t rb = make_rsrc(bin + t0 * H + head, len > 0 ? ((uint32_t)(len - 1) * H + 1) * 2 : 0);
        const int cb = 8 * (tid & 7);
        uint32_t pbr[8];
        for (int j = 0; j < 8; ++j) pbr[j] = __builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)(cb + j) * H * 2, 0, 0);
        const u32x4 g0 = *reinterpret_cast<const u32x4*>(gam + BT + cb), g1 = *reinterpret_cast<const u32x4*>(gam + BT + cb + 4);
        float rs[4];
        for (int i = 0; i < 4; ++i) rs[i] = gam[2 * BT + 16 * i + (tid >> 4)];
        const float gmv = gam[tid];
        float pb[8];
        for (int j = 0; j < 8; ++j) pb[j] = u2f(pbr[j] << 16) * u2f(j < 4 ? g0[j] : g1[j - 4]);
        gm[tid] = gmv;
        tk.commit_h(Kh, HK, tid);
        tk.commit_h_rows(Kgh, HK, tid, rs);
        tt.commit_h_cols(Tgh, HT, tid, pb);
        tp.commit_h(Ph, HT, tid);
    }
    lds_barrier();
    // W = T diag(beta b^G) K, rows of this wave
    {
        f16x8 bt[2];
        for (int is = 0; is < 2; ++is)
            if (is < lo_js) bt[is] = frag_row(Tgh, HT, im, 32 * is, G);
        for (int kb = 0; kb < 8; ++kb) {
            f32x4 wv = {0.f, 0.f, 0.f, 0.f};
            for (int is = 0; is < 2; ++is)
                if (is < lo_js) mma_h(wv, frag_col(Kh, HK, 32 * is, 16 * kb, G, n), bt[is]);
            st4h(Wh + im * HK + 16 * kb + 4 * G, wv);
        }
    }
    lds_barrier();
    // A = gamma I - W^T Kg, rows 32w .. 32w+31
    f16* Ac = Aw + ch * (DK * DK);
    const float gL = gm[3 * BT];
    for (int rb2 = 0; rb2 < 2; ++rb2) {
        const int k1 = 32 * w + 16 * rb2 + n;
        f16x8 bw[2];
        for (int js = 0; js < 2; ++js) bw[js] = frag_col(Wh, HK, 32 * js, 32 * w + 16 * rb2, G, n);
        for (int kb = 0; kb < 8; ++kb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int js = 0; js < 2; ++js) mma_h(acc, frag_col(Kgh, HK, 32 * js, 16 * kb, G, n), bw[js]);
            f32x4 x;
            for (int r = 0; r < 4; ++r) x[r] = (k1 == 16 * kb + 4 * G + r ? gL : 0.0f) - acc[r];
            st4h(Ac + k1 * DK + 16 * kb + 4 * G, x);
        }
    }
    // U = Qd - P W, rows of this wave (rows past the chunk end: zero q)
    {
        f16* Uc = Uw + ch * (BT * DK);
        const float bg = gm[BT + im];
        f16x8 bp[2];
        for (int is = 0; is < 2; ++is)
            if (is < lo_js) bp[is] = frag_row(Ph, HT, im, 32 * is, G);
        for (int kb = 0; kb < 8; ++kb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int is = 0; is < 2; ++is)
                if (is < lo_js) mma_h(acc, frag_col(Wh, HK, 32 * is, 16 * kb, G, n), bp[is]);
            const u32x2 qw = qv[kb];
            f32x4 x;
            for (int r = 0; r < 4; ++r) {
                const float qv = u2f(r & 1 ? qw[r >> 1] & 0xffff0000u : qw[r >> 1] << 16);
                x[r] = bg * qv - acc[r];
            }
            st4h(Uc + im * DK + 16 * kb + 4 * G, x);
        }
    }
}

// The sequential pass: one workgroup of eight waves per (unit, head, 16 NCT
// value columns), two waves per SIMD; wave w keeps D for keys 16w .. 16w+15
// in fp32 registers, and its fp16 copy goes to LDS as [column][key] for the
// next chunk's product (double-buffered, so each chunk needs one barrier).
// Waves 0..3 stage the chunk tiles: A, U and dO of chunk c - 1 are loaded
// into their registers while chunk c + 1 is computed and stored to the other
// LDS buffer at the end of chunk c. dh' (D of every chunk) goes to the
// workspace as fp16.
constexpr int DHH = 512;        // threads of the fp16 sequential pass

template <int NCT>
__global__ __launch_bounds__(DHH, 1) void bwd_dh_kernel_h(BwdArgs a, const f16* Aw, const f16* Uw, f16* dHw) {
    constexpr int NC = 16 * NCT, HC = NC + 8;     // columns of the tile, LDS row stride (halves)
    __shared__ __attribute__((aligned(16))) f16 Ah[2][DK * HK];    // A [key'][key]
    __shared__ __attribute__((aligned(16))) f16 Uh[2][BT * HK];    // U [row][key]
    __shared__ __attribute__((aligned(16))) f16 dOh[2][BT * HC];   // dO
    __shared__ __attribute__((aligned(16))) f16 dhT[2][NC * HK];   // D [column][key]

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H;
    // XCD-aware: workgroups are dealt to the 8 XCDs round-robin, so the
    // column tiles of one (unit, head), which read the same chunk tiles, are
    // given grid slots 8 apart and share that XCD's L2
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int tile = slot % (DV / NC), pair = (slot / (DV / NC)) * 8 + xcd;
    if (pair >= a.n_pairs) return;
    const int u = pair / H, head = pair - u * H;
    const UnitInfo ui = uniform(unit_info(a.um, u));
    const int c0 = tile * NC;
    const int64_t uh = (int64_t)u * H + head;
    const bf16* dout = reinterpret_cast<const bf16*>(a.dout);
    const int key0 = 16 * w;
    const bool ld = tid < 256;                   // the threads that stage the chunk tiles

    // D at the unit's end: keys key0 + 4G + r, column 16ct + n
    f32x4 dh[NCT];
    const int b_last = (ui.nch - 1) & 1;
    for (int ct = 0; ct < NCT; ++ct) {
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + 4 * G + r, col = 16 * ct + n;
            dh[ct][r] = a.dht ? a.dht[(uh * DK + key) * DV + c0 + col] : 0.0f;
        }
        st4h(dhT[b_last] + (16 * ct + n) * HK + key0 + 4 * G, dh[ct]);
    }

    TileRegs<f16, DK, DK> pa;
    TileRegs<f16, BT, DK> pu;
    TileRegs<bf16, BT, NC> pd;
    auto prefetch = [&](int cc) {
        if (!ld) return;
        int l = ui.len - cc * BT;
        l = l > BT ? BT : l;
        const int64_t tt = ui.start + (int64_t)cc * BT, chh = (int64_t)(ui.cbase + cc) * H + head;
        pa.issue(Aw + chh * (DK * DK), DK, DK, tid);
        pu.issue(Uw + chh * (BT * DK), DK, BT, tid);
        pd.issue(dout + (tt * H + head) * DV + c0, (int64_t)H * DV, l, tid);
    };
    auto commit = [&](int b) {
        if (!ld) return;
        pa.commit_raw(Ah[b], HK, tid);
        pu.commit_raw(Uh[b], HK, tid);
        pd.commit_h(dOh[b], HC, tid);
    };
    if (ui.nch > 0) {
        prefetch(ui.nch - 1);
        commit(b_last);
        if (ui.nch > 1) prefetch(ui.nch - 2);
    }
    lds_barrier();                                   // the last chunk's tiles and D published

    for (int c = ui.nch - 1; c >= 0; --c) {
        const int64_t ch = (int64_t)(ui.cbase + c) * H + head;
        const int b = c & 1;
        // dh' of this chunk to the workspace
        for (int ct = 0; ct < NCT; ++ct)
            for (int r = 0; r < 4; ++r) dHw[(ch * DK + key0 + 4 * G + r) * DV + c0 + 16 * ct + n] = (f16)dh[ct][r];
        // D' = A D + scale U^T dO, keys key0 .. +15
        {
            f16x8 aa[4], au[2];
            for (int ks = 0; ks < 4; ++ks) aa[ks] = frag_row(Ah[b], HK, key0 + n, 32 * ks, G);
            for (int js = 0; js < 2; ++js) au[js] = frag_col(Uh[b], HK, 32 * js, key0, G, n);
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 ad = {0.f, 0.f, 0.f, 0.f}, ae = ad;
                for (int ks = 0; ks < 4; ++ks) mma_h(ad, aa[ks], frag_row(dhT[b], HK, 16 * ct + n, 32 * ks, G));
                for (int js = 0; js < 2; ++js) mma_h(ae, au[js], frag_col(dOh[b], HC, 32 * js, 16 * ct, G, n));
                for (int r = 0; r < 4; ++r) dh[ct][r] = ad[r] + a.scale * ae[r];
                st4h(dhT[b ^ 1] + (16 * ct + n) * HK + key0 + 4 * G, dh[ct]);
            }
        }
        // chunk c - 1 into the other buffers (last read by chunk c + 1), then
        // the loads of chunk c - 2
        if (c > 0) {
            commit(b ^ 1);
            if (c > 1) prefetch(c - 2);
        }
        lds_barrier();                               // D' and chunk c - 1 published
    }
    if (a.dh0)
        for (int ct = 0; ct < NCT; ++ct)
            for (int r = 0; r < 4; ++r) a.dh0[(uh * DK + key0 + 4 * G + r) * DV + c0 + 16 * ct + n] = dh[ct][r];
}

// Eight waves, two per SIMD: waves w and w + 4 share token rows 16w .. +15.
// Group 0 (waves 0..3) forms Y and v_new and accumulates dP, group 1 forms
// dvn and Z (= dV) and accumulates dTb; each accumulates dQd, dKd and dKg for
// the key tiles kb = 2jj + group and forms their dq, dk columns, and the
// finish's M1, dL and element terms are split between the groups by column
// block. Waves 0..3 stage the tiles.
__global__ __launch_bounds__(512, 1) void bwd_grad_kernel_h(BwdArgs a, const f16* dHw) {
    __shared__ __attribute__((aligned(16))) f16 Kh[BT * HK];
    __shared__ __attribute__((aligned(16))) f16 Qh[BT * HK];
    __shared__ __attribute__((aligned(16))) f16 Th[BT * HT];     // T
    __shared__ __attribute__((aligned(16))) f16 Tbh[BT * HT];    // T diag(beta)
    __shared__ __attribute__((aligned(16))) f16 Ph[BT * HT];
    // value tiles, reused by the finish for three 64 x 64 tiles
    __shared__ __attribute__((aligned(16))) f16 vb[2 * DK * HV + 6 * BT * HV];
    __shared__ __attribute__((aligned(16))) float gm[4 * BT];
    __shared__ float bt[BT], rowG[2][BT], rowK[2][BT], rowB[2][BT], colP[8][BT], colB[4][BT], red[8];
    __shared__ __attribute__((aligned(16))) float dPf[BT * BTL4];   // finish: dP (fp32), from group 0 to both
    f16* Hh = vb;                       // h      [key][col]
    f16* DHh = Hh + DK * HV;            // dh'    [key][col]
    f16* Vh = DHh + DK * HV;            // v      [row][col]
    f16* DOh = Vh + BT * HV;            // dO
    f16* DVh = DOh + BT * HV;           // dvn
    f16* Yh = DVh + BT * HV;            // Y
    f16* VNh = Yh + BT * HV;            // v_new
    f16* Zh = VNh + BT * HV;            // Z
    f16* X1h = vb;                      // finish: dTb, then beta dL o D
    f16* X2h = vb + BT * HT;            // finish: dP o D
    f16* M1h = vb + 2 * BT * HT;        // finish: dT T^T
    static_assert(3 * BT * HT <= 2 * DK * HV + 6 * BT * HV, "finish tiles fit the value-tile buffers");

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6), w = w8 & 3, grp = w8 >> 2;
    const bool ld = tid < 256;                  // the threads that stage tiles
    const int ci = blockIdx.x, head = blockIdx.y, H = a.H;
    int u, cc;
    chunk_of(a.um, ci, u, cc);
    if (u < 0) return;
    const UnitInfo ui = unit_info(a.um, u);
    const int64_t t0 = ui.start + (int64_t)cc * BT;
    int len = ui.len - cc * BT;
    len = len < 0 ? 0 : (len > BT ? BT : len);
    const int64_t ch = (int64_t)ci * H + head;
    const float lnb = a.use_exp2 ? 0.6931471805599453f : 1.0f;
    const bf16* vin = reinterpret_cast<const bf16*>(a.v);
    const bf16* dout = reinterpret_cast<const bf16*>(a.dout);
    const bf16* bin = reinterpret_cast<const bf16*>(a.beta);
    const int row0 = 16 * w, im = row0 + n;     // this lane's token row in the transposed products
    const int lo_js = w >= 2 ? 2 : 1;           // 32-row steps j <= i can reach
    const int hi_js = w >= 2 ? 1 : 0;           // first 32-row step j >= i can reach

    // the value tiles of tile vt + 1 are loaded into registers while tile vt
    // is computed, and written to LDS at the next tile's top
    TileRegs<float, DK, HVT> ph;
    TileRegs<f16, DK, HVT> pdh;
    TileRegs<bf16, BT, HVT> pv, pdo;
    auto prefetch = [&](int vt) {
        if (!ld) return;
        const int vc0 = vt * HVT;
        ph.issue(a.h + ch * DK * DV + vc0, DV, DK, tid);
        pdh.issue(dHw + ch * DK * DV + vc0, DV, DK, tid);
        pv.issue(vin + (t0 * H + head) * DV + vc0, (int64_t)H * DV, len, tid);
        pdo.issue(dout + (t0 * H + head) * DV + vc0, (int64_t)H * DV, len, tid);
    };
    if (ld) {
        TileRegs<bf16, BT, DK> tk, tq;
        TileRegs<f16, BT, BT> tt, tp;               // T and P: fp16 from the preparation
        const int64_t rs = (int64_t)H * DK;
        tk.issue(reinterpret_cast<const bf16*>(a.k) + (t0 * H + head) * DK, rs, len, tid);
        tq.issue(reinterpret_cast<const bf16*>(a.q) + (t0 * H + head) * DK, rs, len, tid);
        tt.issue(reinterpret_cast<const f16*>(a.ws.Tm) + ch * (BT * BT), BT, BT, tid);
        tp.issue(reinterpret_cast<const f16*>(a.ws.P) + ch * (BT * BT), BT, BT, tid);
        // raw bf16 beta (past the chunk end zero), converted after the value
        // tile loads are issued: a conversion next to its load would wait
        // for every load before it
        const rsrc_t rb = make_rsrc(bin + t0 * H + head, len > 0 ? ((uint32_t)(len - 1) * H + 1) * 2 : 0);
        const int cb = 8 * (tid & 7);                // this thread's T columns 8 (tid & 7) + j
        uint32_t pbr[8];
        for (int j = 0; j < 8; ++j) pbr[j] = __builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)(cb + j) * H * 2, 0, 0);
        const uint32_t btr = __builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)(tid & (BT - 1)) * H * 2, 0, 0);
        const float gmv = a.ws.gam[ch * (GAMR * BT) + tid];   // G, b^G, b^{G_L - G}, b^{G_L}
        prefetch(0);
        float pb[8];
        for (int j = 0; j < 8; ++j) pb[j] = u2f(pbr[j] << 16);
        if (tid < BT) bt[tid] = u2f(btr << 16);
        gm[tid] = gmv;
        tk.commit_h(Kh, HK, tid);
        tq.commit_h(Qh, HK, tid);
        tt.commit_h(Th, HT, tid, pb, Tbh);
        tp.commit_h(Ph, HT, tid);
    }

    // accumulators, transposed: lane (G, n) holds row im at columns 16 b + 4G + r;
    // aPT is dP (group 0) or dTb (group 1), the others key tile 2jj + grp
    f32x4 aPT[4], aQ[4], aKg[4], aKd[4];
    for (int j = 0; j < 4; ++j) {
        aPT[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        aQ[j] = aPT[j];
        aKg[j] = aPT[j];
        aKd[j] = aPT[j];
    }
    float hdh = 0.0f;                                // this thread's share of sum(h o dh')

    for (int vt = 0; vt < DV / HVT; ++vt) {
        const int vc0 = vt * HVT;
        lds_barrier();                               // the previous tile's buffers are consumed
        if (ld) {
            ph.commit_h(Hh, HV, tid);
            pdh.commit_raw(DHh, HV, tid);
            pv.commit_h(Vh, HV, tid);
            pdo.commit_h(DOh, HV, tid);
        }
        lds_barrier();
        if (ld) {
            // this thread's share of sum(h o dh'): its fp32 h against the fp16 dh'
#pragma unroll
            for (int i = 0; i < TileRegs<float, DK, HVT>::PT; ++i) {
                const int e = tid + 256 * i, r = e / 8, c4 = (e % 8) * 4;
                const f32x4 d4 = ld4h(DHh + r * HV + c4);
                for (int j = 0; j < 4; ++j) hdh += u2f(ph.w[i][j]) * d4[j];
            }
        }
        if (vt + 1 < DV / HVT) prefetch(vt + 1);
        // group 0: Y = V - b^G (K h); group 1: dvn = b^{G_L - G} (K dh') + scale P^T dO; rows of this wave
        {
            f16x8 bk[4], bp[2];
            for (int ks = 0; ks < 4; ++ks) bk[ks] = frag_row(Kh, HK, im, 32 * ks, G);
            if (grp == 1)
                for (int js = 0; js < 2; ++js)
                    if (js >= hi_js) bp[js] = frag_col(Ph, HT, 32 * js, row0, G, n);
            for (int mb = 0; mb < 2; ++mb) {
                if (grp == 0) {
                    const float bg = gm[BT + im];
                    f32x4 kh = {0.f, 0.f, 0.f, 0.f};
                    for (int ks = 0; ks < 4; ++ks) mma_h(kh, frag_col(Hh, HV, 32 * ks, 16 * mb, G, n), bk[ks]);
                    const f32x4 v4 = ld4h(Vh + im * HV + 16 * mb + 4 * G);
                    f32x4 y;
                    for (int r = 0; r < 4; ++r) y[r] = v4[r] - bg * kh[r];
                    st4h(Yh + im * HV + 16 * mb + 4 * G, y);
                } else {
                    const float blg = gm[2 * BT + im];
                    f32x4 kd = {0.f, 0.f, 0.f, 0.f}, pd = kd;
                    for (int ks = 0; ks < 4; ++ks) mma_h(kd, frag_col(DHh, HV, 32 * ks, 16 * mb, G, n), bk[ks]);
                    for (int js = 0; js < 2; ++js)
                        if (js >= hi_js) mma_h(pd, frag_col(DOh, HV, 32 * js, 16 * mb, G, n), bp[js]);
                    f32x4 dv;
                    for (int r = 0; r < 4; ++r) dv[r] = blg * kd[r] + a.scale * pd[r];
                    st4h(DVh + im * HV + 16 * mb + 4 * G, dv);
                }
            }
        }
        lds_barrier();
        // group 0: v_new = Tb Y; group 1: Z = Tb^T dvn = dV; rows of this wave
        if (grp == 0) {
            f16x8 btb[2];
            for (int js = 0; js < 2; ++js)
                if (js < lo_js) btb[js] = frag_row(Tbh, HT, im, 32 * js, G);
            for (int mb = 0; mb < 2; ++mb) {
                f32x4 vn = {0.f, 0.f, 0.f, 0.f};
                for (int js = 0; js < 2; ++js)
                    if (js < lo_js) mma_h(vn, frag_col(Yh, HV, 32 * js, 16 * mb, G, n), btb[js]);
                st4h(VNh + im * HV + 16 * mb + 4 * G, vn);
            }
        } else {
            f16x8 btt[2];
            for (int js = 0; js < 2; ++js)
                if (js >= hi_js) btt[js] = frag_col(Th, HT, 32 * js, row0, G, n);
            const float bi = bt[im];
            for (int mb = 0; mb < 2; ++mb) {
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                for (int js = 0; js < 2; ++js)
                    if (js >= hi_js) mma_h(z, frag_col(DVh, HV, 32 * js, 16 * mb, G, n), btt[js]);
                for (int r = 0; r < 4; ++r) z[r] *= bi;
                st4h(Zh + im * HV + 16 * mb + 4 * G, z);
                if (im < len) *reinterpret_cast<f32x4*>(a.dv + ((t0 + im) * H + head) * DV + vc0 + 16 * mb + 4 * G) = z;
            }
        }
        lds_barrier();
        // accumulate over this tile's 32 columns: dP / scale (group 0) or dTb
        // (group 1), and dQd / scale, dKg and -dKd of key tiles 2jj + grp;
        // the wave's rows as n
        {
            const f16x8 bdo = frag_row(DOh, HV, im, 0, G), bvn = frag_row(VNh, HV, im, 0, G);
            const f16x8 bz = frag_row(Zh, HV, im, 0, G);
            const f16x8 bpt = grp == 0 ? bdo : frag_row(DVh, HV, im, 0, G);
            const f16* xpt = grp == 0 ? VNh : Yh;
            for (int jb = 0; jb < 4; ++jb)
                if (jb <= w) mma_h(aPT[jb], frag_row(xpt, HV, 16 * jb + n, 0, G), bpt);
            for (int jj = 0; jj < 4; ++jj) {
                const int kb = 2 * jj + grp;
                const f16x8 hk = frag_row(Hh, HV, 16 * kb + n, 0, G);
                mma_h(aQ[jj], hk, bdo);
                mma_h(aKd[jj], hk, bz);
                mma_h(aKg[jj], frag_row(DHh, HV, 16 * kb + n, 0, G), bvn);
            }
        }
    }
    lds_barrier();

    // ---- finish. X1 = dTb (group 1, fp16), dPf = dP (group 0, fp32), lower
    // incl. diagonal, of the wave's rows; dbeta's column term: sums over i of
    // dTb o T
    {
        float cs[16];                                // value 4 jb + r: column j = 16 jb + 4G + r
        for (int jb = 0; jb < 4; ++jb) {
            const f32x4 t4 = ld4h(Th + im * HT + 16 * jb + 4 * G);
            f32x4 x;
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jb + 4 * G + r;
                const bool keep = jb <= w && j <= im;
                x[r] = keep ? (grp == 0 ? a.scale : 1.0f) * aPT[jb][r] : 0.0f;
                cs[4 * jb + r] = x[r] * t4[r];
            }
            if (grp == 0) *reinterpret_cast<f32x4*>(&dPf[im * BTL4 + 16 * jb + 4 * G]) = x;
            else st4h(X1h + im * HT + 16 * jb + 4 * G, x);
        }
        // lane n: the column sum over this wave's rows of value n
        const float csum = row_sum16(cs, n);
        if (grp == 1) colB[w][16 * (n >> 2) + 4 * G + (n & 3)] = csum;
    }
    lds_barrier();
    // M1 = dT T^T = dTb Tb^T, rows of this wave, column blocks 2 grp, 2 grp + 1
    {
        f16x8 bx[2];
        for (int js = 0; js < 2; ++js)
            if (js < lo_js) bx[js] = frag_row(X1h, HT, im, 32 * js, G);
        for (int kh2 = 0; kh2 < 2; ++kh2) {
            const int kb = 2 * grp + kh2;
            f32x4 m = {0.f, 0.f, 0.f, 0.f};
            for (int js = 0; js < 2; ++js)
                if (js < lo_js) mma_h(m, frag_row(Tbh, HT, 16 * kb + n, 32 * js, G), bx[js]);
            st4h(M1h + im * HT + 16 * kb + 4 * G, m);
        }
    }
    lds_barrier();
    // dL = -T^T M1 (strictly lower) and the Gram matrix K K^T, rows of this
    // wave, column blocks 2 grp, 2 grp + 1
    f32x4 dl[2], gr[2];
    {
        f16x8 btt[2], bk[4];
        for (int js = 0; js < 2; ++js)
            if (js >= hi_js) btt[js] = frag_col(Th, HT, 32 * js, row0, G, n);
        for (int ks = 0; ks < 4; ++ks) bk[ks] = frag_row(Kh, HK, im, 32 * ks, G);
        for (int jh = 0; jh < 2; ++jh) {
            const int jb = 2 * grp + jh;
            dl[jh] = f32x4{0.f, 0.f, 0.f, 0.f};
            gr[jh] = dl[jh];
            if (jb <= w) {
                for (int js = 0; js < 2; ++js)
                    if (js >= hi_js) mma_h(dl[jh], frag_col(M1h, HT, 32 * js, 16 * jb, G, n), btt[js]);
                for (int ks = 0; ks < 4; ++ks) mma_h(gr[jh], frag_row(Kh, HK, 16 * jb + n, 32 * ks, G), bk[ks]);
            }
        }
    }
    // element terms of L and P in column blocks 2 grp, 2 grp + 1: dbeta_i +=
    // sum_j dL_ij G_ij, the G_i / G_j parts of the gate gradient, and dG o D,
    // dP o D into X1, X2
    float rg = 0.0f;
    {
        const float gi = gm[im], bi = bt[im];
        float rb = 0.0f, cg[16];
        for (int e = 0; e < 16; ++e) cg[e] = 0.0f;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            if ((jb >> 1) != grp) continue;          // (jb static, so cg stays in registers)
            const int jh = jb & 1;
            const f32x4 p4 = ld4h(Ph + im * HT + 16 * jb + 4 * G);
            const f32x4 dp4 = *reinterpret_cast<const f32x4*>(&dPf[im * BTL4 + 16 * jb + 4 * G]);
            f32x4 x1, x2;
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jb + 4 * G + r;
                const float d = jb <= w && j <= im ? fpow(gi - gm[j], a.use_exp2) : 0.0f;
                const float lij = j < im ? -dl[jh][r] : 0.0f;     // dL
                const float gij = gr[jh][r] * d;                   // (k_i . k_j) D_ij
                const float dgg = bi * lij;                        // dG
                const float dpij = dp4[r];
                rb += lij * gij;
                const float t = lnb * (dgg * gij + dpij * p4[r]);
                rg += t;
                cg[4 * jb + r] = -t;
                x1[r] = dgg * d;
                x2[r] = dpij * d;
            }
            st4h(X1h + im * HT + 16 * jb + 4 * G, x1);
            st4h(X2h + im * HT + 16 * jb + 4 * G, x2);
        }
        // row sums over the four lane groups
        rb = pair32(pair16(rb));
        rg = pair32(pair16(rg));
        if (G == 0) rowB[grp][im] = rb;
        // column sums over this wave's rows: one partial per wave, added in a
        // fixed order below (the same result on every run)
        colP[w8][16 * (n >> 2) + 4 * G + (n & 3)] = row_sum16(cg, n);
    }
    lds_barrier();
    // dq, dk, rows of this wave and key tiles 2jj + grp: the products with
    // dG o D and dP o D, then b^G dQd, b^G dKd + b^{G_L - G} dKg, and their
    // gate terms
    {
        f16x8 x2r[2], x1r[2], x1c[2], x2c[2];
        for (int js = 0; js < 2; ++js) {
            if (js < lo_js) {
                x2r[js] = frag_row(X2h, HT, im, 32 * js, G);
                x1r[js] = frag_row(X1h, HT, im, 32 * js, G);
            }
            if (js >= hi_js) {
                x1c[js] = frag_col(X1h, HT, 32 * js, row0, G, n);
                x2c[js] = frag_col(X2h, HT, 32 * js, row0, G, n);
            }
        }
        const float bgi = gm[BT + im], blgi = gm[2 * BT + im];
        float rq = 0.0f, rk = 0.0f;
        for (int jj = 0; jj < 4; ++jj) {
            const int kb = 2 * jj + grp;
            f32x4 q1 = {0.f, 0.f, 0.f, 0.f}, k1 = q1;
            for (int js = 0; js < 2; ++js) {
                const f16x8 ak = frag_col(Kh, HK, 32 * js, 16 * kb, G, n);
                if (js < lo_js) {
                    mma_h(q1, ak, x2r[js]);
                    mma_h(k1, ak, x1r[js]);
                }
                if (js >= hi_js) {
                    mma_h(k1, ak, x1c[js]);
                    mma_h(k1, frag_col(Qh, HK, 32 * js, 16 * kb, G, n), x2c[js]);
                }
            }
            const f32x4 q4 = ld4h(Qh + im * HK + 16 * kb + 4 * G), k4 = ld4h(Kh + im * HK + 16 * kb + 4 * G);
            f32x4 dqv, dkv;
            for (int r = 0; r < 4; ++r) {
                const float dQd = a.scale * aQ[jj][r], dKd = -aKd[jj][r], dKg = aKg[jj][r];
                dqv[r] = q1[r] + bgi * dQd;
                dkv[r] = k1[r] + bgi * dKd + blgi * dKg;
                // the Kg term (ln b dKg Kg) goes to dg as a prefix over earlier
                // rows: its - part here and its + part in G_L's gradient cancel
                // for every row from i on
                rq += lnb * (dQd * bgi * q4[r] + dKd * bgi * k4[r]);
                rk += lnb * dKg * blgi * k4[r];
            }
            if (im < len) {
                const int64_t o = ((t0 + im) * H + head) * DK + 16 * kb + 4 * G;
                *reinterpret_cast<f32x4*>(a.dq + o) = dqv;
                *reinterpret_cast<f32x4*>(a.dk + o) = dkv;
            }
        }
        rq = pair32(pair16(rq));
        rk = pair32(pair16(rk));
        if (G == 0) {
            rowG[grp][im] = rg + rq;
            rowK[grp][im] = rk;
        }
    }
    // the state decay's term of G_L: lnb gamma sum(h o dh'), over the workgroup
    float tl = lnb * gm[3 * BT] * hdh;
    for (int sft = 1; sft < 64; sft <<= 1) tl += __shfl_xor(tl, sft, 64);
    if (lane == 0) red[w8] = tl;
    lds_barrier();
    // dg: reverse cumulative sum over the chunk's rows of the gate gradient,
    // with the state decay's term entering at the last valid row, plus the
    // exclusive prefix of the Kg terms; dbeta: its column and row terms
    if (w8 == 0) {
        float gl = 0.0f, colG = 0.0f, colBs = 0.0f;
        for (int i = 0; i < 8; ++i) {
            gl += red[i];
            colG += colP[i][lane];
        }
        for (int i = 0; i < 4; ++i) colBs += colB[i][lane];
        float x = lane < len ? (rowG[0][lane] + rowG[1][lane]) + colG + (lane == len - 1 ? gl : 0.0f) : 0.0f;
        const float kg = lane < len ? rowK[0][lane] + rowK[1][lane] : 0.0f;
        float y = kg;
        for (int sft = 1; sft < 64; sft <<= 1) {
            const float xd = __shfl_down(x, sft, 64), yu = __shfl_up(y, sft, 64);
            if (lane + sft < 64) x += xd;
            if (lane >= sft) y += yu;
        }
        x += y - kg;
        if (lane < len) {
            a.dg[(t0 + lane) * H + head] = x;
            a.dbeta[(t0 + lane) * H + head] = colBs + rowB[0][lane] + rowB[1][lane];
        }
    }
}

// ------------------------------------------------------------------ launcher
hipError_t launch_bwd(const Problem& p, const Workspace& ws, float* dH, float* dVN, const void* q, const void* k,
                      const void* v, const float* g, const void* beta, const float* h, const void* dout,
                      const float* dht, float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                      bool dh_only, bool reuse_prep, hipStream_t s) {
    if (!reuse_prep && launch_prep_bwd(p, ws, k, q, g, beta, s) != hipSuccess) return hipGetLastError();
    // bf16 inputs, scalar gate: dh' as fp16 in the first half of the dH
    // region and U in the second, A in the dvn region (the grad kernel forms
    // dvn itself)
    const bool h16 = p.dtype == 1 && !p.per_key;
    const int64_t nchh = (int64_t)p.um.n_chunks * p.H;
    f16* dHw = reinterpret_cast<f16*>(dH);
    f16* Uw = dHw + nchh * DK * DV;
    f16* Aw = reinterpret_cast<f16*>(dVN);
    // per key: A (fp32) in the dvn region, U^T over the Qd tiles
    float* Ak = dVN;
    BwdArgs a;
    a.um = p.um; a.H = p.H; a.use_exp2 = p.use_exp2; a.scale = p.scale;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g; a.dout = dout; a.h = h; a.dht = dht;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    a.ws = ws; a.dH = dH; a.dVN = dVN;
    a.n_pairs = p.um.n_units * p.H;
    if (!reuse_prep && p.um.n_chunks > 0) {
        const dim3 grid(p.um.n_chunks, p.H);
        if (h16) hipLaunchKernelGGL(bwd_transfer_kernel_h, grid, dim3(256), 0, s, a, Aw, Uw);
        else if (p.per_key && p.dtype == 1) hipLaunchKernelGGL(bwd_transfer_kernel_pk<bf16>, grid, dim3(256), 0, s, a, Ak);
        else if (p.per_key) hipLaunchKernelGGL(bwd_transfer_kernel_pk<float>, grid, dim3(256), 0, s, a, Ak);
    }
    if (a.n_pairs > 0) {
        // 32-column tiles while they fill the compute units, else 16-column
        // tiles (twice the workgroups, half the products per step)
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipGetLastError();
        const bool narrow = 4 * (int64_t)a.n_pairs < cus;
        const dim3 grid((narrow ? 8 : 4) * 8 * ((a.n_pairs + 7) / 8));
        // per key (one workgroup per compute unit): the narrowest tiles whose
        // workgroups all run at once, else 64-column tiles
        const int pk_nct = 8 * (int64_t)a.n_pairs <= cus ? 1 : 4 * (int64_t)a.n_pairs <= cus ? 2 : 4;
        const dim3 grid_pk((DV / (16 * pk_nct)) * 8 * ((a.n_pairs + 7) / 8));
#define GDN_DHA(IN)                                                                                   \
    if (pk_nct == 4) hipLaunchKernelGGL((bwd_dh_kernel_pkr<IN, 4>), grid_pk, dim3(PKR), 0, s, a, Ak); \
    else if (pk_nct == 2) hipLaunchKernelGGL((bwd_dh_kernel_pkr<IN, 2>), grid_pk, dim3(PKR), 0, s, a, Ak); \
    else hipLaunchKernelGGL((bwd_dh_kernel_pkr<IN, 1>), grid_pk, dim3(PKR), 0, s, a, Ak);
        if (p.per_key) {
            if (p.dtype == 1) { GDN_DHA(bf16) } else { GDN_DHA(float) }
        } else if (h16) {
            if (narrow) hipLaunchKernelGGL(bwd_dh_kernel_h<1>, grid, dim3(DHH), 0, s, a, Aw, Uw, dHw);
            else hipLaunchKernelGGL(bwd_dh_kernel_h<2>, grid, dim3(DHH), 0, s, a, Aw, Uw, dHw);
        } else if (narrow) {
            hipLaunchKernelGGL(bwd_dh_kernel<1>, grid, dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL(bwd_dh_kernel<2>, grid, dim3(256), 0, s, a);
        }
#undef GDN_DHA
    }
    if (p.um.n_chunks > 0 && !dh_only) {
        dim3 grid(p.um.n_chunks, p.H);
        if (p.per_key) {
            if (p.dtype == 1) {
                hipLaunchKernelGGL(bwd_grad_kernel_pk<bf16>, grid, dim3(512), 0, s, a);
            } else {
                hipLaunchKernelGGL(bwd_grad_kernel_pk<float>, grid, dim3(512), 0, s, a);
            }
        } else {
            if (p.dtype == 1) hipLaunchKernelGGL(bwd_grad_kernel_h, grid, dim3(512), 0, s, a, dHw);
            else hipLaunchKernelGGL(bwd_grad_kernel, grid, dim3(256), 0, s, a);
        }
    }
    return hipGetLastError();
}

}  // namespace gdn
