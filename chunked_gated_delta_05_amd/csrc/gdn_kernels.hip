// HIP kernels of the chunkwise gated delta rule forward for gfx950 (CDNA4).
//
// Chunk form (one unit, one head, one chunk of n <= 64 tokens, entry state h
// in K x V, G_i the chunk-local inclusive cumulative gate, b the decay base):
//
//   L_ij   = beta_i (k_i . k_j) b^{G_i - G_j}           j < i
//            (per key: beta_i sum_d k_id k_jd b^{G_id - G_jd})
//   T      = (I + L)^{-1}                              unit lower triangular
//   Y_i    = beta_i (v_i - (k_i * b^{G_i}) h)          the residual before the solve
//   v_new  = T Y                                        (the u - w h of the WY form)
//   o_i    = scale [ (q_i * b^{G_i}) h + sum_{j<=i} P_ij v_new_j ],
//            P_ij = (q_i . k_j) b^{G_i - G_j}  (per key: sum_d q_id k_jd b^{G_id - G_jd})
//   h_next = Diag(b^{G_last}) h + sum_j (k_j * b^{G_last - G_j}) v_new_j^T
//
// v_new = T Y is the product u - w h with u = T diag(beta) V and
// w = T diag(beta) (K * b^G) regrouped, so neither w nor u is ever stored: the
// preparation kernel keeps only T. The inter-chunk recurrence is the one of
// kda_split_state_summary_kernel on the state_summary.py coverage page
// (residual first, then the decayed state plus the gated-key update).
//
// Kernels:
//   prep_kernel   one workgroup per (chunk, head): G, L on MFMA, the 64 x 64
//                 triangular inverse in LDS, T to the workspace (per-key gate:
//                 also P, q*b^G, k*b^G, k*b^{G_last-G}, G_last).
//   state_kernel  one workgroup per (unit, head, 32-column value tile): walks
//                 the unit's chunks with the 128 x 32 fp32 state tile in
//                 registers, fused with the output; in summary mode it runs
//                 the same recurrence on [S_ext | M] from [0 | I].
//   merge_kernel  S_init[s+1] = M_s S_init[s] + S_ext[s] in fp32.
//
// Precision: every MFMA takes bf16 operands with fp32 accumulation. Operands
// that are not exact bf16 values (the state, the residual Y, v_new, P, and on
// the per-key path the gated q and k) are split into hi + lo bf16 pairs and
// multiplied as hi*hi + hi*lo + lo*hi, which keeps the o path at about 16
// significant bits; the fp32 input path uses fp32 MFMA throughout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ float bpow(float x, int use_exp2) { return use_exp2 ? exp2f(x) : expf(x); }
// b^x with the hardware base-2 exponential (about 1 ulp; e^x = 2^(x log2 e))
__device__ __forceinline__ float fpow(float x, int use_exp2) {
    return __builtin_amdgcn_exp2f(use_exp2 ? x : x * 1.4426950408889634f);
}

// ------------------------------------------------------------------ policies
// A fragment holds, for lane (G = lane / 16, n = lane % 16), the 8 elements
// X[n][8G .. 8G+7] of a 16 x 32 A tile or X[8G .. 8G+7][n] of a 32 x 16 B
// tile: the operand layout of v_mfma_f32_16x16x32_bf16. The accumulator holds
// C[4G + r][n], r = 0..3.

struct PolicyBF16 {
    using In = bf16;
    static constexpr int PLANES = 2;
    struct F { bf16x8 v; };
    struct S { bf16x8 hi, lo; };

    __device__ static F ldF(const In* p) { F f; f.v = *reinterpret_cast<const bf16x8*>(p); return f; }
    __device__ static F zeroF() { F f; for (int e = 0; e < 8; ++e) f.v[e] = (bf16)0.0f; return f; }
    __device__ static F roundF(const float* x) {
        F f;
        for (int e = 0; e < 8; ++e) f.v[e] = (bf16)x[e];
        return f;
    }
    __device__ static S splitS(const float* x) {
        S s;
        for (int e = 0; e < 8; ++e) {
            bf16 h = (bf16)x[e];
            s.hi[e] = h;
            s.lo[e] = (bf16)(x[e] - (float)h);
        }
        return s;
    }
    __device__ static S zeroS() { S s; F z = zeroF(); s.hi = z.v; s.lo = z.v; return s; }
    // four consecutive values into a hi/lo plane pair (ps = plane stride in elements)
    __device__ static void st4(In* p, int ps, const float* x) {
        bf16x4 h, l;
        for (int e = 0; e < 4; ++e) {
            h[e] = (bf16)x[e];
            l[e] = (bf16)(x[e] - (float)h[e]);
        }
        *reinterpret_cast<bf16x4*>(p) = h;
        *reinterpret_cast<bf16x4*>(p + ps) = l;
    }
    __device__ static S ldS(const In* p, int64_t ps) {
        S s;
        s.hi = *reinterpret_cast<const bf16x8*>(p);
        s.lo = *reinterpret_cast<const bf16x8*>(p + ps);
        return s;
    }
    __device__ static void mma(f32x4& c, const bf16x8& a, const bf16x8& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static void mFF(f32x4& c, const F& a, const F& b) { mma(c, a.v, b.v); }
    __device__ static void mFS(f32x4& c, const F& a, const S& b) { mma(c, a.v, b.hi); mma(c, a.v, b.lo); }
    __device__ static void mSF(f32x4& c, const S& a, const F& b) { mma(c, a.hi, b.v); mma(c, a.lo, b.v); }
    __device__ static void mSS(f32x4& c, const S& a, const S& b) {
        mma(c, a.hi, b.hi);
        mma(c, a.hi, b.lo);
        mma(c, a.lo, b.hi);
    }
    // Column fragment of an LDS tile: lane (G, n) gets tile[r0 + 8G + e][c0 + n].
    // ds_read_b64_tr_b16 hands component c of lane j's 4-element row to lane
    // 4(j%4)+c as element j/4, so lane j points at row r0 + 8G + j/4 (+4),
    // columns c0 + 4(j%4) .. +3.
    __device__ static bf16x8 ldcol_raw(const In* tile, int ld, int r0, int c0, int lane) {
        const int G = lane >> 4, j = lane & 15;
        const In* p = tile + (r0 + 8 * G + (j >> 2)) * ld + c0 + 4 * (j & 3);
        s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p));
        s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p + 4 * ld));
        bf16x4 x = __builtin_bit_cast(bf16x4, a), y = __builtin_bit_cast(bf16x4, b);
        bf16x8 r;
        for (int e = 0; e < 4; ++e) { r[e] = x[e]; r[e + 4] = y[e]; }
        return r;
    }
    __device__ static F ldcolF(const In* tile, int ld, int r0, int c0, int lane) {
        F f; f.v = ldcol_raw(tile, ld, r0, c0, lane); return f;
    }
    __device__ static S ldcolS(const In* tile, int ps, int ld, int r0, int c0, int lane) {
        S s;
        s.hi = ldcol_raw(tile, ld, r0, c0, lane);
        s.lo = ldcol_raw(tile + ps, ld, r0, c0, lane);
        return s;
    }
    __device__ static float f(In x) { return (float)x; }
    __device__ static In cvt(float x) { return (bf16)x; }
};

struct PolicyF32 {
    using In = float;
    static constexpr int PLANES = 1;
    struct F { float v[8]; };
    using S = F;

    __device__ static F ldF(const In* p) {
        F f;
        f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
        for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[e + 4] = b[e]; }
        return f;
    }
    __device__ static F zeroF() { F f; for (int e = 0; e < 8; ++e) f.v[e] = 0.0f; return f; }
    __device__ static F roundF(const float* x) { F f; for (int e = 0; e < 8; ++e) f.v[e] = x[e]; return f; }
    __device__ static S splitS(const float* x) { return roundF(x); }
    __device__ static S zeroS() { return zeroF(); }
    __device__ static void st4(In* p, int, const float* x) {
        f32x4 a;
        for (int e = 0; e < 4; ++e) a[e] = x[e];
        *reinterpret_cast<f32x4*>(p) = a;
    }
    __device__ static S ldS(const In* p, int64_t) { return ldF(p); }
    // the 32-deep product as eight 16x16x4 fp32 MFMAs: instruction e takes
    // element e of every lane, so together they cover k = 8G + e for all G, e
    __device__ static void m8(f32x4& c, const F& a, const F& b) {
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    }
    __device__ static void mFF(f32x4& c, const F& a, const F& b) { m8(c, a, b); }
    __device__ static void mFS(f32x4& c, const F& a, const S& b) { m8(c, a, b); }
    __device__ static void mSF(f32x4& c, const S& a, const F& b) { m8(c, a, b); }
    __device__ static void mSS(f32x4& c, const S& a, const S& b) { m8(c, a, b); }
    __device__ static F ldcolF(const In* tile, int ld, int r0, int c0, int lane) {
        const int G = lane >> 4, n = lane & 15;
        F f;
        for (int e = 0; e < 8; ++e) f.v[e] = tile[(r0 + 8 * G + e) * ld + c0 + n];
        return f;
    }
    __device__ static S ldcolS(const In* tile, int, int ld, int r0, int c0, int lane) {
        return ldcolF(tile, ld, r0, c0, lane);
    }
    __device__ static float f(In x) { return x; }
    __device__ static In cvt(float x) { return x; }
};

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
        r.start = (int64_t)u * um.T;
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

// ------------------------------------------------------------------ prep
constexpr int LDK = DK + 8;   // row stride of 64 x 128 LDS tiles (elements)
constexpr int LDL = BT + 1;   // row stride of 64 x 64 fp32 LDS matrices

struct PrepArgs {
    UnitMap um;
    int H;
    const void* k;
    const void* q;       // per-key only
    const float* g;
    const void* beta;
    int use_exp2;
    Workspace ws;
    float* g_cumsum;     // optional slot, token-major
    float* A;            // optional slot, token-major [tokens][H][64]
};

template <class P, bool PERKEY>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    using In = typename P::In;
    __shared__ __attribute__((aligned(16))) In kt[BT * LDK];
    __shared__ __attribute__((aligned(16))) In qt[PERKEY ? BT * LDK : 8];
    __shared__ float Gs[PERKEY ? BT * (DK + 4) : BT];
    __shared__ float bet[BT];
    __shared__ float Ls[BT * LDL];
    __shared__ float Ts[BT * LDL];
    __shared__ float Yb[3 * 16 * 17];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, G = lane >> 4, n = lane & 15;
    const int ci = blockIdx.x, head = blockIdx.y, H = a.H;
    int u, cc;
    chunk_of(a.um, ci, u, cc);
    if (u < 0) return;
    const UnitInfo ui = unit_info(a.um, u);
    const int64_t t0 = ui.start + (int64_t)cc * BT;
    int len = ui.len - cc * BT;
    len = len < 0 ? 0 : (len > BT ? BT : len);
    const int64_t ch = (int64_t)ci * H + head;   // chunk-head index into the workspace
    const In* kin = reinterpret_cast<const In*>(a.k);
    const In* qin = reinterpret_cast<const In*>(a.q);
    const In* bin = reinterpret_cast<const In*>(a.beta);
    const bool has_q = PERKEY && qin != nullptr;   // per key: prepare q * b^G and P as well

    // ---- tiles into LDS (rows past the chunk end are zero)
    constexpr int VPR = 16 / sizeof(In);             // elements per 16-byte vector
    constexpr int NV = BT * DK / VPR;                // vectors per tile
    for (int idx = tid; idx < NV; idx += 256) {
        const int r = idx / (DK / VPR), cv = (idx % (DK / VPR)) * VPR;
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 kv = z, qv = z;
        if (r < len) {
            kv = *reinterpret_cast<const f32x4*>(kin + ((t0 + r) * H + head) * DK + cv);
            if (has_q) qv = *reinterpret_cast<const f32x4*>(qin + ((t0 + r) * H + head) * DK + cv);
        }
        *reinterpret_cast<f32x4*>(&kt[r * LDK + cv]) = kv;
        if (PERKEY) *reinterpret_cast<f32x4*>(&qt[r * LDK + cv]) = qv;
    }
    if (tid < BT) bet[tid] = tid < len ? P::f(bin[(t0 + tid) * H + head]) : 0.0f;
    if (!PERKEY) {
        // inclusive scan of the scalar gate over the chunk, one wave
        if (w == 0) {
            float x = lane < len ? a.g[(t0 + lane) * H + head] : 0.0f;
            for (int off = 1; off < 64; off <<= 1) {
                float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            Gs[lane] = x;
            a.ws.gam[ch * BT + lane] = x;
            if (a.g_cumsum && lane < len) a.g_cumsum[(t0 + lane) * H + head] = x;
        }
    } else {
        // per-key gate: running sum down each key column
        if (tid < DK) {
            float acc = 0.0f;
            for (int r = 0; r < BT; ++r) {
                if (r < len) acc += a.g[((t0 + r) * H + head) * DK + tid];
                Gs[r * (DK + 4) + tid] = acc;
                if (a.g_cumsum && r < len) a.g_cumsum[((t0 + r) * H + head) * DK + tid] = acc;
            }
            a.ws.gamL[ch * DK + tid] = acc;
        }
    }
    __syncthreads();

    // ---- L = strictly lower (beta_i k_i.k_j b^{G_i-G_j}) on MFMA, 10 tiles over 4 waves
    {
        const int mid = len > 0 ? (len - 1) / 2 : 0;   // reference row of the per-key factorisation
        for (int t = w; t < 10; t += 4) {
            const int it = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            const int jt = t - (it * (it + 1)) / 2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < DK / 32; ++kk) {
                const int col = 32 * kk + 8 * G;
                if (!PERKEY) {
                    typename P::F A = P::ldF(&kt[(16 * it + n) * LDK + col]);
                    typename P::F B = P::ldF(&kt[(16 * jt + n) * LDK + col]);
                    P::mFF(acc, A, B);
                } else {
                    float xa[8], xb[8];
                    for (int e = 0; e < 8; ++e) {
                        const float gr = Gs[mid * (DK + 4) + col + e];
                        xa[e] = P::f(kt[(16 * it + n) * LDK + col + e]) *
                                bpow(Gs[(16 * it + n) * (DK + 4) + col + e] - gr, a.use_exp2);
                        xb[e] = P::f(kt[(16 * jt + n) * LDK + col + e]) *
                                bpow(gr - Gs[(16 * jt + n) * (DK + 4) + col + e], a.use_exp2);
                    }
                    P::mSS(acc, P::splitS(xa), P::splitS(xb));
                }
            }
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * G + r, j = 16 * jt + n;
                float l = 0.0f;
                if (j < i) {
                    l = bet[i] * acc[r];
                    if (!PERKEY) l *= bpow(Gs[i] - Gs[j], a.use_exp2);
                }
                Ls[i * LDL + j] = l;
            }
        }
    }
    __syncthreads();

    // ---- T = (I + L)^{-1}: 16 x 16 diagonal blocks by substitution (wave 0,
    // lane = block * 16 + column), then the off-diagonal blocks by distance
    if (w == 0) {
        const int bk = lane >> 4, c = lane & 15, o = 16 * bk;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < i; ++j) s += Ls[(o + i) * LDL + o + j] * x[j];
            x[i] = i == c ? 1.0f : (i > c ? -s : 0.0f);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Ts[(o + i) * LDL + o + c] = x[i];
    } else {
        // zero the blocks above the diagonal
        for (int e = tid - 64; e < 6 * 256; e += 192) {
            const int blk = e >> 8, rr = (e >> 4) & 15, cc2 = e & 15;
            const int I = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
            const int J = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
            Ts[(16 * I + rr) * LDL + 16 * J + cc2] = 0.0f;
        }
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        const int nb = 4 - d;
        for (int e = tid; e < nb * 256; e += 256) {
            const int bi = e >> 8, rr = (e >> 4) & 15, cc2 = e & 15;
            const int I = d + bi, J = bi;
            float s = 0.0f;
            for (int K2 = J; K2 < I; ++K2)
                for (int m = 0; m < 16; ++m)
                    s += Ls[(16 * I + rr) * LDL + 16 * K2 + m] * Ts[(16 * K2 + m) * LDL + 16 * J + cc2];
            Yb[(bi * 16 + rr) * 17 + cc2] = s;
        }
        __syncthreads();
        for (int e = tid; e < nb * 256; e += 256) {
            const int bi = e >> 8, rr = (e >> 4) & 15, cc2 = e & 15;
            const int I = d + bi, J = bi;
            float s = 0.0f;
            for (int m = 0; m < 16; ++m) s += Ts[(16 * I + rr) * LDL + 16 * I + m] * Yb[(bi * 16 + m) * 17 + cc2];
            Ts[(16 * I + rr) * LDL + 16 * J + cc2] = -s;
        }
        __syncthreads();
    }

    // ---- T out (row-major 64 x 64 fp32), optional token-major A slot
    float* Tw = a.ws.Tm + ch * (BT * BT);
    for (int e = tid; e < BT * BT / 4; e += 256) {
        const int r = e / (BT / 4), c4 = (e % (BT / 4)) * 4;
        f32x4 x;
        for (int q2 = 0; q2 < 4; ++q2) x[q2] = Ts[r * LDL + c4 + q2];
        *reinterpret_cast<f32x4*>(Tw + r * BT + c4) = x;
        if (a.A && r < len) *reinterpret_cast<f32x4*>(a.A + ((t0 + r) * H + head) * BT + c4) = x;
    }

    if (PERKEY) {
        // P = q.k decayed, lower triangle with the diagonal; stored fp32 row-major
        const int mid = len > 0 ? (len - 1) / 2 : 0;
        float* Pw = a.ws.P + ch * (BT * BT);
        for (int t = w; has_q && t < 16; t += 4) {
            const int it = t >> 2, jt = t & 3;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (jt <= it) {
                for (int kk = 0; kk < DK / 32; ++kk) {
                    const int col = 32 * kk + 8 * G;
                    float xa[8], xb[8];
                    for (int e = 0; e < 8; ++e) {
                        const float gr = Gs[mid * (DK + 4) + col + e];
                        xa[e] = P::f(qt[(16 * it + n) * LDK + col + e]) *
                                bpow(Gs[(16 * it + n) * (DK + 4) + col + e] - gr, a.use_exp2);
                        xb[e] = P::f(kt[(16 * jt + n) * LDK + col + e]) *
                                bpow(gr - Gs[(16 * jt + n) * (DK + 4) + col + e], a.use_exp2);
                    }
                    P::mSS(acc, P::splitS(xa), P::splitS(xb));
                }
            }
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * G + r, j = 16 * jt + n;
                Pw[i * BT + j] = j <= i ? acc[r] : 0.0f;
            }
        }
        // gated q and k tiles: q*b^G (split), k*b^G (one plane), k*b^{G_last-G} (split)
        const int64_t plane = a.ws.plane;
        In* qg = reinterpret_cast<In*>(a.ws.qg) + ch * (BT * DK);
        In* kd = reinterpret_cast<In*>(a.ws.kd) + ch * (BT * DK);
        In* kg = reinterpret_cast<In*>(a.ws.kg) + ch * (BT * DK);
        const int last = len > 0 ? len - 1 : 0;
        for (int e4 = tid; e4 < BT * DK / 4; e4 += 256) {
            const int r = e4 / (DK / 4), c4 = (e4 % (DK / 4)) * 4;
            float xq[4], xd[4], xg[4];
            for (int e = 0; e < 4; ++e) {
                const float gg = Gs[r * (DK + 4) + c4 + e];
                const float kv = P::f(kt[r * LDK + c4 + e]);
                xq[e] = P::f(qt[r * LDK + c4 + e]) * bpow(gg, a.use_exp2);
                xd[e] = kv * bpow(gg, a.use_exp2);
                xg[e] = kv * bpow(Gs[last * (DK + 4) + c4 + e] - gg, a.use_exp2);
            }
            if (has_q) P::st4(qg + r * DK + c4, (int)plane, xq);
            P::st4(kg + r * DK + c4, (int)plane, xg);
            for (int e = 0; e < 4; ++e) kd[r * DK + c4 + e] = P::cvt(xd[e]);
        }
    }
}

// ------------------------------------------------------------------ state pass
constexpr int LDH = DK + 8;   // hT rows (value column) of 128 keys
constexpr int LDY = BT + 8;   // YT / vnT rows (value column) of 64 tokens

struct StateArgs {
    UnitMap um;
    int H;
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    Workspace ws;
    const float* h0;
    void* o;
    int o_bf16;
    float* hfinal;
    float* hslot;
    float scale;
    int use_exp2;
    int n_pairs;     // units * H
    int ntiles;      // column tiles per pair
    int tile0;       // first column tile (summary mode: 0, or V / 32 for M only)
    float* S_ext;
    float* M;
};

template <class P, bool PERKEY, bool SUMMARY>
__global__ __launch_bounds__(256) void state_kernel(StateArgs a) {
    using In = typename P::In;
    using F = typename P::F;
    using S = typename P::S;
    constexpr int NP = P::PLANES;
    __shared__ __attribute__((aligned(16))) In kt[2][BT * LDK];                   // k (per key: k*b^G)
    __shared__ __attribute__((aligned(16))) In kgt[PERKEY ? NP * BT * LDK : 8];  // per key: k*b^{G_last-G}
    __shared__ __attribute__((aligned(16))) In hT[NP * BV * LDH];                // state, transposed
    __shared__ __attribute__((aligned(16))) In YT[NP * BV * LDY];
    __shared__ __attribute__((aligned(16))) In vnT[NP * BV * LDY];
    __shared__ __attribute__((aligned(16))) In vpT[NP * BV * LDY];
    __shared__ __attribute__((aligned(16))) In PS[(!PERKEY && !SUMMARY) ? 4 * NP * 16 * LDY : 8];
    __shared__ float gam[2][BT];
    __shared__ float bet[2][BT];
    __shared__ float gl[2][PERKEY ? DK : 1];

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept scalar
    const int H = a.H;
    // blocks are dealt round-robin to the 8 XCDs: keep every column tile of a
    // (unit, head) pair on one XCD so that they share its L2
    const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
    const int tile = slot % a.ntiles + a.tile0;
    const int pair = (slot / a.ntiles) * 8 + xcd;
    if (pair >= a.n_pairs) return;
    const int u = pair / H, head = pair - u * H;
    const UnitInfo ui = unit_info(a.um, u);
    const int c0 = tile * BV;                       // column of [S_ext | M] or of V
    const bool mcols = SUMMARY && c0 >= DV;         // transfer-map columns: v = 0, start at I
    const int vc0 = mcols ? c0 - DV : c0;
    const In* qin = reinterpret_cast<const In*>(a.q);
    const In* kin = reinterpret_cast<const In*>(a.k);
    const In* vin = reinterpret_cast<const In*>(a.v);
    const In* bin = reinterpret_cast<const In*>(a.beta);
    const int nkw = w >= 2 ? 2 : 1;                  // 32-token steps that cover rows <= 16w+15
    const int e2 = a.use_exp2;

    // ---- state tile: rows (keys) 32w + 16ks + 4G + r, columns vc0 + 16vs + n
    f32x4 h[2][2];
    for (int ks = 0; ks < 2; ++ks)
        for (int vs = 0; vs < 2; ++vs)
            for (int r = 0; r < 4; ++r) {
                const int key = 32 * w + 16 * ks + 4 * G + r, col = vc0 + 16 * vs + n;
                float x = 0.0f;
                if (mcols) x = key == col ? 1.0f : 0.0f;
                else if (!SUMMARY && a.h0) x = a.h0[(((int64_t)u * H + head) * DK + key) * DV + col];
                h[ks][vs][r] = x;
            }

    // ---- next-chunk prefetch. Loads stay raw in registers until the chunk is
    // used one step later, so their latency overlaps a whole step; rows past
    // the chunk end read a clamped (valid) row and are zeroed at use.
    constexpr int VPR = 16 / sizeof(In);
    constexpr int NKV = BT * DK / VPR / 256;          // 16-byte vectors per thread for a 64 x 128 tile
    auto chunk_len = [&](int c) { int l = ui.len - c * BT; return l < 0 ? 0 : (l > BT ? BT : l); };
    struct Raw {
        f32x4 k[NKV];    // k tile (per key: k*b^G), 16-byte vectors
        float gb;        // thread < 64: G; 128..255: G_last per key
        In bt;           // thread 64..127: beta
        F q[4];          // scalar gate: q rows 16w+n
        S qs[4];         // per-key gate: q*b^G rows 16w+n
        f32x4 T[2][2];   // T rows 16w+n, columns 32kk + 8G .. +7
        f32x4 Pw[2][2];  // per-key gate: P rows 16w+n
        In v[2][4];      // v rows 16w+4G+r, columns vc0+16vs+n
        f32x4 kg[PERKEY ? NP : 1][NKV];   // per-key gate: k*b^{G_last-G} tile planes
        int len;
    };
    auto load_raw = [&](int c, Raw& x) {
        const int len = chunk_len(c);
        x.len = len;
        const int last = len > 0 ? len - 1 : 0;
        const int64_t t0 = ui.start + (int64_t)c * BT;
        const int64_t ch = (int64_t)(ui.cbase + c) * H + head;
        for (int i = 0; i < NKV; ++i) {
            const int idx = tid + 256 * i, r = idx / (DK / VPR), cv = (idx % (DK / VPR)) * VPR;
            if (PERKEY) x.k[i] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const In*>(a.ws.kd) + ch * (BT * DK) + r * DK + cv);
            else x.k[i] = *reinterpret_cast<const f32x4*>(kin + ((t0 + min(r, last)) * H + head) * DK + cv);
        }
        // every thread loads (no divergent branches around loads); publish keeps
        // what its wave owns: wave 0 G, wave 1 beta, waves 2-3 G_last per key
        x.gb = PERKEY ? a.ws.gamL[ch * DK + (tid & (DK - 1))] : a.ws.gam[ch * BT + lane];
        x.bt = bin[(t0 + min(lane, last)) * H + head];
        if (PERKEY) {
            const In* src = reinterpret_cast<const In*>(a.ws.kg) + ch * (BT * DK);
            for (int p = 0; p < NP; ++p)
                for (int i = 0; i < NKV; ++i) {
                    const int idx = tid + 256 * i, r = idx / (DK / VPR), cv = (idx % (DK / VPR)) * VPR;
                    x.kg[p][i] = *reinterpret_cast<const f32x4*>(src + p * a.ws.plane + r * DK + cv);
                }
        }
        const int row = 16 * w + n;
        if (!SUMMARY) {
            if (!PERKEY) {
                const In* qr = qin + ((t0 + min(row, last)) * H + head) * DK + 8 * G;
                for (int kk = 0; kk < 4; ++kk) x.q[kk] = P::ldF(qr + 32 * kk);
            } else {
                const In* qg = reinterpret_cast<const In*>(a.ws.qg) + ch * (BT * DK) + row * DK + 8 * G;
                for (int kk = 0; kk < 4; ++kk) x.qs[kk] = P::ldS(qg + 32 * kk, a.ws.plane);
                const float* Pr = a.ws.P + ch * (BT * BT) + row * BT + 8 * G;
                for (int kk = 0; kk < 2; ++kk)
                    if (kk < nkw) {
                        x.Pw[kk][0] = *reinterpret_cast<const f32x4*>(Pr + 32 * kk);
                        x.Pw[kk][1] = *reinterpret_cast<const f32x4*>(Pr + 32 * kk + 4);
                    }
            }
        }
        const float* Tr = a.ws.Tm + ch * (BT * BT) + row * BT + 8 * G;
        for (int kk = 0; kk < 2; ++kk)
            if (kk < nkw) {
                x.T[kk][0] = *reinterpret_cast<const f32x4*>(Tr + 32 * kk);
                x.T[kk][1] = *reinterpret_cast<const f32x4*>(Tr + 32 * kk + 4);
            }
        if (!mcols)
            for (int r = 0; r < 4; ++r) {
                const In* vr = vin + ((t0 + min(16 * w + 4 * G + r, last)) * H + head) * DV + vc0 + n;
                x.v[0][r] = vr[0];
                x.v[1][r] = vr[16];
            }
    };
    // chunk data that the whole workgroup reads through LDS
    auto publish = [&](const Raw& x, int b) {
        for (int i = 0; i < NKV; ++i) {
            const int idx = tid + 256 * i, r = idx / (DK / VPR), cv = (idx % (DK / VPR)) * VPR;
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4*>(&kt[b][r * LDK + cv]) = r < x.len ? x.k[i] : z;
        }
        if (w == 0) { if (!PERKEY) gam[b][lane] = x.gb; }
        else if (w == 1) bet[b][lane] = lane < x.len ? P::f(x.bt) : 0.0f;
        else if (PERKEY) gl[b][tid - 2 * BT] = x.gb;
    };
    auto t_frag = [&](const Raw& x, int kk) {
        float f[8];
        for (int e = 0; e < 4; ++e) { f[e] = x.T[kk][0][e]; f[e + 4] = x.T[kk][1][e]; }
        return P::roundF(f);
    };

    // ---- prologue
    const int nch = ui.nch;
    Raw cur, nxt;
    if (nch > 0) {
        load_raw(0, cur);
        publish(cur, 0);
    }
    if (!PERKEY && !SUMMARY) {
        // columns of the wave's P rows that are never computed stay zero
        for (int e = lane; e < NP * 16 * LDY; e += 64) PS[w * NP * 16 * LDY + e] = P::cvt(0.0f);
    }
    for (int ks = 0; ks < 2; ++ks)
        for (int vs = 0; vs < 2; ++vs) {
            float x[4] = {h[ks][vs][0], h[ks][vs][1], h[ks][vs][2], h[ks][vs][3]};
            P::st4(&hT[(16 * vs + n) * LDH + 32 * w + 16 * ks + 4 * G], BV * LDH, x);
        }
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        const int len = cur.len;
        const int64_t t0 = ui.start + (int64_t)c * BT;
        const bool more = c + 1 < nch;
        if (more) load_raw(c + 1, nxt);
        if (PERKEY) {
            // k*b^{G_last-G} of this chunk (prefetched a step ago); the previous
            // chunk's reads of kgt ended before the last barrier, and the reads of
            // this one follow the next two
            for (int p = 0; p < NP; ++p)
                for (int i = 0; i < NKV; ++i) {
                    const int idx = tid + 256 * i, r = idx / (DK / VPR), cv = (idx % (DK / VPR)) * VPR;
                    *reinterpret_cast<f32x4*>(&kgt[p * BT * LDK + r * LDK + cv]) = cur.kg[p][i];
                }
        }
        if (!SUMMARY && a.hslot) {
            for (int ks = 0; ks < 2; ++ks)
                for (int vs = 0; vs < 2; ++vs)
                    for (int r = 0; r < 4; ++r) {
                        const int key = 32 * w + 16 * ks + 4 * G + r, col = vc0 + 16 * vs + n;
                        a.hslot[(((int64_t)(ui.cbase + c) * H + head) * DK + key) * DV + col] = h[ks][vs][r];
                    }
        }
        // per-row decay factors of this lane's accumulator rows i = 16w + 4G + r
        float eG[4], eLG[4];
        const float gL = PERKEY ? 0.0f : gam[b][len > 0 ? len - 1 : 0];
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * G + r;
            eG[r] = PERKEY ? 1.0f : fpow(gam[b][i], e2);
            eLG[r] = PERKEY ? 1.0f : fpow(gL - gam[b][i], e2);
        }
        const bool qrow = 16 * w + n < len;
        F qa[4];
        if (!SUMMARY && !PERKEY)
            for (int kk = 0; kk < 4; ++kk) qa[kk] = qrow ? cur.q[kk] : P::zeroF();

        // ---- token side: K h and q h for rows 16w .. 16w+15
        const In* K = kt[b];
        f32x4 kh[2], qh[2];
        for (int vs = 0; vs < 2; ++vs) {
            kh[vs] = f32x4{0.f, 0.f, 0.f, 0.f};
            qh[vs] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int kk = 0; kk < 4; ++kk) {
            const F ka = P::ldF(&K[(16 * w + n) * LDK + 32 * kk + 8 * G]);
            for (int vs = 0; vs < 2; ++vs) {
                const S hb = P::ldS(&hT[(16 * vs + n) * LDH + 32 * kk + 8 * G], BV * LDH);
                F hhi;
                if constexpr (NP == 2) hhi.v = hb.hi; else hhi = hb;
                P::mFF(kh[vs], ka, hhi);
                if (!SUMMARY) {
                    if (!PERKEY) P::mFS(qh[vs], qa[kk], hb);
                    else P::mSS(qh[vs], cur.qs[kk], hb);
                }
            }
        }
        // Y = beta (v - b^G K h) (per key: K already carries b^G)
        for (int vs = 0; vs < 2; ++vs) {
            float y[4];
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * G + r;
                const float vv = (!mcols && i < len) ? P::f(cur.v[vs][r]) : 0.0f;
                y[r] = bet[b][i] * (vv - eG[r] * kh[vs][r]);
            }
            P::st4(&YT[(16 * vs + n) * LDY + 16 * w + 4 * G], BV * LDY, y);
        }
        f32x4 oacc[2];
        if (!SUMMARY) {
            for (int vs = 0; vs < 2; ++vs)
                for (int r = 0; r < 4; ++r) oacc[vs][r] = eG[r] * qh[vs][r];
            if (!PERKEY) {
                // P^T tiles (j block jt, i block w): rows j, columns i = 16w + n
                const float gi = gam[b][16 * w + n];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    if (jt > w) continue;
                    f32x4 pt = {0.f, 0.f, 0.f, 0.f};
                    for (int kk = 0; kk < 4; ++kk)
                        P::mFF(pt, P::ldF(&K[(16 * jt + n) * LDK + 32 * kk + 8 * G]), qa[kk]);
                    float x[4];
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * jt + 4 * G + r;
                        x[r] = j <= 16 * w + n ? pt[r] * fpow(gi - gam[b][j], e2) : 0.0f;
                    }
                    P::st4(&PS[w * NP * 16 * LDY + n * LDY + 16 * jt + 4 * G], 16 * LDY, x);
                }
            }
        }
        __syncthreads();

        // ---- v_new = T Y for rows 16w .. 16w+15
        f32x4 vn[2];
        for (int vs = 0; vs < 2; ++vs) vn[vs] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < 2; ++kk) {
            if (kk >= nkw) continue;
            const F ta = t_frag(cur, kk);
            for (int vs = 0; vs < 2; ++vs)
                P::mFS(vn[vs], ta, P::ldS(&YT[(16 * vs + n) * LDY + 32 * kk + 8 * G], BV * LDY));
        }
        for (int vs = 0; vs < 2; ++vs) {
            float x[4], xp[4];
            for (int r = 0; r < 4; ++r) {
                x[r] = vn[vs][r];
                xp[r] = x[r] * eLG[r];
            }
            if (!SUMMARY) P::st4(&vnT[(16 * vs + n) * LDY + 16 * w + 4 * G], BV * LDY, x);
            P::st4(&vpT[(16 * vs + n) * LDY + 16 * w + 4 * G], BV * LDY, xp);
        }
        __syncthreads();

        // ---- output rows 16w .. 16w+15
        if (!SUMMARY) {
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= nkw) continue;
                S pa;
                if (!PERKEY) {
                    pa = P::ldS(&PS[w * NP * 16 * LDY + n * LDY + 32 * kk + 8 * G], 16 * LDY);
                } else {
                    float f[8];
                    for (int e = 0; e < 4; ++e) { f[e] = cur.Pw[kk][0][e]; f[e + 4] = cur.Pw[kk][1][e]; }
                    pa = P::splitS(f);
                }
                for (int vs = 0; vs < 2; ++vs)
                    P::mSS(oacc[vs], pa, P::ldS(&vnT[(16 * vs + n) * LDY + 32 * kk + 8 * G], BV * LDY));
            }
            for (int vs = 0; vs < 2; ++vs)
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * w + 4 * G + r;
                    if (i < len) {
                        const int64_t oi = ((t0 + i) * H + head) * DV + vc0 + 16 * vs + n;
                        const float x = a.scale * oacc[vs][r];
                        if (a.o_bf16) reinterpret_cast<bf16*>(a.o)[oi] = (bf16)x;
                        else reinterpret_cast<float*>(a.o)[oi] = x;
                    }
                }
        }

        // ---- state: h = Diag(b^{G_last}) h + kg^T v_new' for keys 32w .. 32w+31
        S vb[2][2];
        for (int kk = 0; kk < 2; ++kk)
            for (int vs = 0; vs < 2; ++vs)
                vb[kk][vs] = P::ldS(&vpT[(16 * vs + n) * LDY + 32 * kk + 8 * G], BV * LDY);
        const float eL = PERKEY ? 1.0f : fpow(gL, e2);
        for (int ks = 0; ks < 2; ++ks) {
            float dec[4];
            for (int r = 0; r < 4; ++r)
                dec[r] = PERKEY ? fpow(gl[b][32 * w + 16 * ks + 4 * G + r], e2) : eL;
            for (int vs = 0; vs < 2; ++vs)
                for (int r = 0; r < 4; ++r) h[ks][vs][r] *= dec[r];
            for (int kk = 0; kk < 2; ++kk) {
                if (!PERKEY) {
                    const F ka = P::ldcolF(K, LDK, 32 * kk, 32 * w + 16 * ks, lane);
                    for (int vs = 0; vs < 2; ++vs) P::mFS(h[ks][vs], ka, vb[kk][vs]);
                } else {
                    const S ka = P::ldcolS(kgt, BT * LDK, LDK, 32 * kk, 32 * w + 16 * ks, lane);
                    for (int vs = 0; vs < 2; ++vs) P::mSS(h[ks][vs], ka, vb[kk][vs]);
                }
            }
            for (int vs = 0; vs < 2; ++vs) {
                float x[4] = {h[ks][vs][0], h[ks][vs][1], h[ks][vs][2], h[ks][vs][3]};
                P::st4(&hT[(16 * vs + n) * LDH + 32 * w + 16 * ks + 4 * G], BV * LDH, x);
            }
        }
        if (more) {
            publish(nxt, b ^ 1);
            cur = nxt;
        }
        __syncthreads();
    }

    // ---- results
    for (int ks = 0; ks < 2; ++ks)
        for (int vs = 0; vs < 2; ++vs)
            for (int r = 0; r < 4; ++r) {
                const int key = 32 * w + 16 * ks + 4 * G + r, col = vc0 + 16 * vs + n;
                const int64_t uh = (int64_t)u * H + head;
                if (SUMMARY) {
                    if (mcols) { if (a.M) a.M[(uh * DK + key) * DK + col] = h[ks][vs][r]; }
                    else if (a.S_ext) a.S_ext[(uh * DK + key) * DV + col] = h[ks][vs][r];
                } else if (a.hfinal) {
                    a.hfinal[(uh * DK + key) * DV + col] = h[ks][vs][r];
                }
            }
}

// ------------------------------------------------------------------ merge
constexpr int MC = 8;   // state columns per merge workgroup

__global__ __launch_bounds__(256) void merge_kernel(int H, int n_seg, const float* S_ext, const float* M,
                                                     const float* S0, float* S_init, float* S_final) {
    __shared__ float Ms[DK * (DK + 1)];
    __shared__ float Sc[DK * MC];
    const int tid = threadIdx.x, c = tid % MC, rbase = tid / MC;   // rows rbase + 32 i
    const int col0 = blockIdx.x * MC, bh = blockIdx.y, b = bh / H, head = bh % H;
    for (int i = 0; i < 4; ++i) {
        const int r = rbase + 32 * i;
        Sc[r * MC + c] = S0 ? S0[((int64_t)bh * DK + r) * DV + col0 + c] : 0.0f;
    }
    for (int s = 0; s < n_seg; ++s) {
        const int64_t us = ((int64_t)b * n_seg + s) * H + head;
        __syncthreads();
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + 32 * i;
            S_init[(us * DK + r) * DV + col0 + c] = Sc[r * MC + c];
        }
        for (int e = tid; e < DK * DK; e += 256) Ms[(e / DK) * (DK + 1) + e % DK] = M[us * DK * DK + e];
        __syncthreads();
        float acc[4];
        for (int i = 0; i < 4; ++i) acc[i] = S_ext[(us * DK + rbase + 32 * i) * DV + col0 + c];
        for (int m = 0; m < DK; ++m) {
            const float sv = Sc[m * MC + c];
            for (int i = 0; i < 4; ++i) acc[i] += Ms[(rbase + 32 * i) * (DK + 1) + m] * sv;
        }
        __syncthreads();
        for (int i = 0; i < 4; ++i) Sc[(rbase + 32 * i) * MC + c] = acc[i];
    }
    __syncthreads();
    if (S_final)
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + 32 * i;
            S_final[((int64_t)bh * DK + r) * DV + col0 + c] = Sc[r * MC + c];
        }
}

// ------------------------------------------------------------------ launchers
static int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

size_t workspace_bytes(const Problem& p, Workspace* ws, char* base) {
    const int64_t nch = (int64_t)p.um.n_chunks * p.H;
    const int64_t es = p.dtype == 1 ? 2 : 4;
    const int planes = p.dtype == 1 ? 2 : 1;
    int64_t off = 0;
    auto take = [&](int64_t bytes) { int64_t o = off; off = align256(off + bytes); return o; };
    const int64_t oT = take(nch * BT * BT * 4);
    const int64_t og = take(nch * BT * 4);
    int64_t oP = 0, oq = 0, od = 0, ok = 0, ol = 0;
    if (p.per_key) {
        oP = take(nch * BT * BT * 4);
        oq = take(planes * nch * BT * DK * es);
        od = take(nch * BT * DK * es);
        ok = take(planes * nch * BT * DK * es);
        ol = take(nch * DK * 4);
    }
    if (ws && base) {
        ws->Tm = reinterpret_cast<float*>(base + oT);
        ws->gam = reinterpret_cast<float*>(base + og);
        ws->P = p.per_key ? reinterpret_cast<float*>(base + oP) : nullptr;
        ws->qg = p.per_key ? base + oq : nullptr;
        ws->kd = p.per_key ? base + od : nullptr;
        ws->kg = p.per_key ? base + ok : nullptr;
        ws->gamL = p.per_key ? reinterpret_cast<float*>(base + ol) : nullptr;
        ws->plane = nch * BT * DK;
    }
    return (size_t)(off > 0 ? off : 256);
}

hipError_t launch_prep(const Problem& p, const Workspace& ws, const void* k, const void* q,
                       const float* g, const void* beta, float* g_cumsum_slot, float* A_slot,
                       hipStream_t s) {
    if (p.um.n_chunks == 0) return hipSuccess;
    PrepArgs a;
    a.um = p.um; a.H = p.H; a.k = k; a.q = q; a.g = g; a.beta = beta; a.use_exp2 = p.use_exp2;
    a.ws = ws; a.g_cumsum = g_cumsum_slot; a.A = A_slot;
    dim3 grid(p.um.n_chunks, p.H), block(256);
    if (p.dtype == 1) {
        if (p.per_key) hipLaunchKernelGGL((prep_kernel<PolicyBF16, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prep_kernel<PolicyBF16, false>), grid, block, 0, s, a);
    } else {
        if (p.per_key) hipLaunchKernelGGL((prep_kernel<PolicyF32, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prep_kernel<PolicyF32, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <class P, bool PK>
static void launch_state_t(bool summary, dim3 grid, hipStream_t s, const StateArgs& a) {
    if (summary) hipLaunchKernelGGL((state_kernel<P, PK, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((state_kernel<P, PK, false>), grid, dim3(256), 0, s, a);
}

hipError_t launch_state(const Problem& p, const Workspace& ws, const void* q, const void* k,
                        const void* v, const void* beta, const float* h0, void* o, float* hfinal,
                        float* hslot, int summary, int want_ext, int want_M, float* S_ext,
                        float* M, hipStream_t s) {
    StateArgs a;
    a.um = p.um; a.H = p.H; a.q = q; a.k = k; a.v = v; a.beta = beta; a.ws = ws;
    a.h0 = h0; a.o = o; a.o_bf16 = p.o_dtype == 1; a.hfinal = hfinal; a.hslot = hslot;
    a.scale = p.scale; a.use_exp2 = p.use_exp2;
    a.n_pairs = p.um.n_units * p.H;
    a.S_ext = S_ext; a.M = M;
    if (summary) {
        a.tile0 = want_ext ? 0 : DV / BV;
        a.ntiles = (want_ext ? DV / BV : 0) + (want_M ? DK / BV : 0);
    } else {
        a.tile0 = 0;
        a.ntiles = DV / BV;
    }
    if (a.n_pairs == 0 || a.ntiles == 0) return hipSuccess;
    const int groups = (a.n_pairs + 7) / 8;
    dim3 grid(8 * a.ntiles * groups);
    if (p.dtype == 1) {
        if (p.per_key) launch_state_t<PolicyBF16, true>(summary, grid, s, a);
        else launch_state_t<PolicyBF16, false>(summary, grid, s, a);
    } else {
        if (p.per_key) launch_state_t<PolicyF32, true>(summary, grid, s, a);
        else launch_state_t<PolicyF32, false>(summary, grid, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_merge(int B, int H, int n_seg, const float* S_ext, const float* M,
                        const float* S0, float* S_init, float* S_final, hipStream_t s) {
    if (B * H == 0) return hipSuccess;
    dim3 grid(DV / MC, B * H);
    hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, s, H, n_seg, S_ext, M, S0, S_init, S_final);
    return hipGetLastError();
}

}  // namespace gdn
