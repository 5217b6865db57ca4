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
//   prep_kernel_h    bf16, scalar gate: one wave per (chunk, head) with every
//                    tile in registers: G, L and P on MFMA, the 64 x 64 inverse
//                    (diagonal blocks by substitution, the rest on fp32 MFMA),
//                    T diag(beta), P and the per-row coefficients to the
//                    workspace.
//   prep_kernel_pk   bf16, per-key gate: four waves per (chunk, head); the
//                    gated operands computed once per element, L and P on
//                    MFMA, the inverse in LDS.
//   prep_kernel      fp32 inputs (scalar and per-key gates): one workgroup per
//                    (chunk, head), the inverse in LDS (per-key gate: also
//                    q*b^G, k*b^G, k*b^{G_last-G}, G_last).
//   state_kernel_ks  bf16, scalar and per-key gates: one workgroup per (unit,
//                    head, 32 columns); four compute waves split the state by
//                    keys, four streaming waves stage the chunk tiles (per key:
//                    the prepared gated k, q and k b^{G_L - G} tiles).
//   state_kernel     fp32 inputs: eight waves, each owning 32 keys of 16
//                    columns. In summary mode every state kernel runs the same
//                    recurrence on [S_ext | M] from [0 | I].
//   merge_kernel     S_init[s+1] = M_s S_init[s] + S_ext[s] in fp32.
//   unit_order_kernel  packed units ranked by chunk count, so that the state
//                    passes launch the longest units first.
//
// The bf16 scalar-gate preparation writes T diag(beta) (the A slot keeps T),
// so the state pass needs no beta.
//
// Precision: bf16 inputs are converted to fp16 MFMA operands (exact for
// normal-range values); products accumulate in fp32; the state, the cumulative
// gates and the triangular solve stay fp32, and operands computed on the fly
// (the state, the residual Y, v_new, P, T) are rounded to fp16 once. fp32
// inputs use fp32 MFMA throughout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdn_internal.h"
#include "gdn_device.h"

namespace gdn {

// ------------------------------------------------------------------ policies
// A fragment holds, for lane (G = lane / 16, n = lane % 16), the 8 elements
// X[n][8G .. 8G+7] of a 16 x 32 A tile or X[8G .. 8G+7][n] of a 32 x 16 B
// tile: the operand layout of v_mfma_f32_16x16x32_{f16,bf16}. The
// accumulator holds C[4G + r][n], r = 0..3.

struct PolicyH {          // fp16 operands (bf16 inputs)
    using Op = f16;
    struct F { f16x8 v; };
    __device__ static F ld(const Op* p) { F f; f.v = *reinterpret_cast<const f16x8*>(p); return f; }
    __device__ static void st4(Op* p, const float* x) {
        f16x4 h;
        for (int e = 0; e < 4; ++e) h[e] = (f16)x[e];
        *reinterpret_cast<f16x4*>(p) = h;
    }
    __device__ static void mma(f32x4& c, const F& a, const F& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
    }
    // 4 fp32 values -> 4 operands (8 bytes)
    __device__ static void f32_to_op4(Op* p, f32x4 x) {
        f16x4 h;
        for (int e = 0; e < 4; ++e) h[e] = (f16)x[e];
        *reinterpret_cast<f16x4*>(p) = h;
    }
};

struct PolicyF {          // fp32 inputs and operands
    using In = float;
    using Op = float;
    static constexpr int LDQ = 132;   // 64 x 128 LDS tile rows: 528 bytes
    struct F { float v[8]; };
    __device__ static F ld(const Op* p) {
        F f;
        f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
        for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[e + 4] = b[e]; }
        return f;
    }
    __device__ static F from(const float* x) { F f; for (int e = 0; e < 8; ++e) f.v[e] = x[e]; return f; }
    __device__ static void st4(Op* p, const float* x) {
        f32x4 a;
        for (int e = 0; e < 4; ++e) a[e] = x[e];
        *reinterpret_cast<f32x4*>(p) = a;
    }
    // the 32-deep product as eight 16x16x4 fp32 MFMAs: instruction e takes
    // element e of every lane, so together they cover k = 8G + e for all G, e
    __device__ static void mma(f32x4& c, const F& a, const F& b) {
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    }
    __device__ static F ldcol(const Op* tile, int ld, int r0, int c0, int lane) {
        const int G = lane >> 4, n = lane & 15;
        F f;
        for (int e = 0; e < 8; ++e) f.v[e] = tile[(r0 + 8 * G + e) * ld + c0 + n];
        return f;
    }
    __device__ static float f(In x) { return x; }
    __device__ static Op cvt(float x) { return x; }
    static constexpr int FV = 2;   // 16-byte vectors per 8-operand fragment
    __device__ static F frag(const f32x4* v) {
        F f;
        for (int e = 0; e < 4; ++e) { f.v[e] = v[0][e]; f.v[e + 4] = v[1][e]; }
        return f;
    }
    __device__ static f32x4 in2op(f32x4 raw) { return raw; }
    __device__ static void f32_to_op4(Op* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
    // one 16-byte vector of inputs (4 values) -> fp32
    static constexpr int VPR = 4;
    __device__ static void load16(const In* p, float* x) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p);
        for (int e = 0; e < 4; ++e) x[e] = v[e];
    }
};

// ------------------------------------------------------------------ operand order
// Order of the 64 x 128 k / q tiles (along keys) and of the 64 x 64 T and P
// tiles (along tokens) in the fp16 state pass: within each 32-wide slice,
// position 8g + 4h + c holds element 16h + 4g + c. A 16-byte fragment read
// at position 32s + 8g then pairs, element for element, with accumulator
// rows 4g + c of the 16-row tiles 2s (h = 0) and 2s + 1 (h = 1), so that
// accumulators serve as MFMA B operands straight from registers: the order
// of the terms inside one 32-deep contraction does not change the product.
__device__ __forceinline__ int op_pos(int x) { return (x & ~31) | ((x & 12) << 1) | ((x & 16) >> 2) | (x & 3); }

// 16-byte granule swizzle of the 64-operand rows (8 granules) of the T and P
// tiles in LDS. The LDS has 32 four-byte banks: a 16-byte read is served 8
// lanes at a time, so the granule index modulo 8 picks the banks, and the
// row-fragment reads of 8 consecutive rows are conflict free.
__device__ __forceinline__ int swz8(int r) { return r & 7; }

// k and q tiles of the scalar-gate state pass (rows of 16 granules): row r
// keeps logical granule g at g ^ swzk(r), and every odd granule with its two
// 8-byte halves swapped. swzk is a bijection on any 8 consecutive rows (the
// 16-byte row-fragment reads stay conflict free), and on every aligned group
// of 4 rows its bits 0 and 2 take all four values, so a transposed read -
// 4 rows x 4 granules, 8 bytes each, half of them in the swapped halves -
// meets all 32 banks once. A row-fragment read of granule 4s + G lands in
// lanes of group G, so only odd groups see the swapped halves; the state
// operand those reads pair with swaps the same halves on the same lanes,
// which keeps every product's key pairing.
__device__ __forceinline__ int swzk(int r) { return (r & 1) | ((r & 2) << 1) | ((r & 4) >> 1) | (r & 8); }

// Per-chunk coefficient block of the per-key fp16 state pass (CFB bytes,
// written by the preparation): four 64-entry fp16 rows in lane order (entry
// 16G + 4it + r belongs to token row 16it + 4G + r) - beta, 1, 1, beta - then
// the fp32 b^{G_L} of every key.
constexpr int CF_CY = 0, CF_CP = 64, CF_BG = 128, CF_BETA = 192;   // fp16 offsets
constexpr int CF_GL = 128;                                          // fp32 offset
// The scalar gate's block (CFS bytes) holds, at the float offsets below,
// b^{G_L} (one float) and three fp32 rows in the same lane order:
// b^{G_L - G} r_k (the update), b^G r_k (k.h) and b^G r_q (q.h), r being the
// reciprocal q / k norm of the row (1 without normalisation); beta is folded
// into T. Floats 1..63 are not used.
constexpr int CS_EL = 0, CS_CP = 64, CS_BG = 128, CS_BQ = 192;
__device__ __forceinline__ int lane_order(int t) { return 16 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3); }


// ------------------------------------------------------------------ prep
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
    int qk_norm;         // q and k L2-normalised (rows scaled by r = 1 / |x|)
    int beta_sig;        // beta through a sigmoid
    void* q_hat;         // optional slots: the transformed inputs (input dtype) and r
    void* k_hat;
    float* q_rstd;
    float* k_rstd;
    void* beta_eff;
};

template <class P, bool PERKEY>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    using In = typename P::In;
    using Op = typename P::Op;
    constexpr int LDQ = P::LDQ;
    __shared__ __attribute__((aligned(16))) Op kt[BT * LDQ];
    __shared__ __attribute__((aligned(16))) Op qt[BT * LDQ];
    __shared__ float Gs[PERKEY ? BT * (DK + 4) : BT];
    __shared__ float bet[BT];
    __shared__ float Ls[BT * LDL];
    __shared__ float Ts[BT * LDL];
    __shared__ float Yb[3 * 16 * 17];
    __shared__ float Rn[2 * BT];          // reciprocal norms of the k rows, then the q rows

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
    const bool has_q = qin != nullptr;   // P (and per key q * b^G) are prepared when q is given
    // the fp32 path: operands stay in natural order (the fp16 paths have kernels of their own)
    static_assert(sizeof(Op) == 4, "prep_kernel serves fp32 operands");

    // ---- tiles into LDS as operands (rows past the chunk end are zero)
    constexpr int VPR = P::VPR;                      // elements per 16-byte vector
    constexpr int NV = BT * DK / VPR;                // vectors per tile
    for (int idx = tid; idx < NV; idx += 256) {
        const int r = idx / (DK / VPR), cv = (idx % (DK / VPR)) * VPR;
        float kv[VPR], qv[VPR];
        for (int e = 0; e < VPR; ++e) { kv[e] = 0.0f; qv[e] = 0.0f; }
        if (r < len) {
            P::load16(kin + ((t0 + r) * H + head) * DK + cv, kv);
            if (has_q) P::load16(qin + ((t0 + r) * H + head) * DK + cv, qv);
        }
        for (int e = 0; e < VPR; e += 4) {
            *reinterpret_cast<f32x4*>(&kt[r * LDQ + cv + e]) = f32x4{kv[e], kv[e + 1], kv[e + 2], kv[e + 3]};
            *reinterpret_cast<f32x4*>(&qt[r * LDQ + cv + e]) = f32x4{qv[e], qv[e + 1], qv[e + 2], qv[e + 3]};
        }
    }
    // ---- input transforms: k and q rows normalised in place (r = 1 / |x|),
    // beta through a sigmoid; optional slots of the transformed inputs
    __syncthreads();
    if (tid < 2 * BT) {
        const int r = tid & (BT - 1);
        const Op* t = tid < BT ? kt : qt;
        float ss = 0.0f;
        if (a.qk_norm && r < len)
            for (int d = 0; d < DK; ++d) ss += (float)t[r * LDQ + d] * (float)t[r * LDQ + d];
        Rn[tid] = a.qk_norm && r < len ? rnorm_f(ss) : 1.0f;
    }
    __syncthreads();
    if (a.qk_norm || a.k_hat || a.q_hat) {
        for (int e = tid; e < BT * DK; e += 256) {
            const int r = e / DK, d = e % DK;
            const float xk = (float)kt[r * LDQ + d] * Rn[r], xq = (float)qt[r * LDQ + d] * Rn[BT + r];
            if (a.qk_norm) {
                kt[r * LDQ + d] = (Op)xk;
                qt[r * LDQ + d] = (Op)xq;
            }
            if (r < len) {
                if (a.k_hat) reinterpret_cast<In*>(a.k_hat)[((t0 + r) * H + head) * DK + d] = (In)xk;
                if (has_q && a.q_hat) reinterpret_cast<In*>(a.q_hat)[((t0 + r) * H + head) * DK + d] = (In)xq;
            }
        }
    }
    if (tid < len) {
        if (a.k_rstd) a.k_rstd[(t0 + tid) * H + head] = Rn[tid];
        if (has_q && a.q_rstd) a.q_rstd[(t0 + tid) * H + head] = Rn[BT + tid];
    }
    if (tid < BT) {
        float bt = tid < len ? P::f(bin[(t0 + tid) * H + head]) : 0.0f;
        if (a.beta_sig && tid < len) bt = sigmoid_f(bt);
        if (a.beta_eff && tid < len) reinterpret_cast<In*>(a.beta_eff)[(t0 + tid) * H + head] = (In)bt;
        bet[tid] = bt;
    }
    if (!PERKEY) {
        // inclusive scan of the scalar gate over the chunk, one wave; stores
        // G, b^G, b^{G_last - G} and b^{G_last} for the state pass
        if (w == 0) {
            float x = lane < len ? a.g[(t0 + lane) * H + head] : 0.0f;
            for (int off = 1; off < 64; off <<= 1) {
                float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            const float xl = __shfl(x, len > 0 ? len - 1 : 0, 64);
            Gs[lane] = x;
            float* gw = a.ws.gam + ch * (GAMR * BT);
            const float bG = fpow(x, a.use_exp2), bLG = fpow(xl - x, a.use_exp2), bL = fpow(xl, a.use_exp2);
            gw[lane] = x;
            gw[BT + lane] = bG * Rn[lane];
            gw[2 * BT + lane] = bLG * Rn[lane];
            gw[3 * BT + lane] = bL;
            gw[4 * BT + lane] = bG * Rn[BT + lane];
            if (a.g_cumsum && lane < len) a.g_cumsum[(t0 + lane) * H + head] = x;
        }
    } else {
        // per-key gate: the chunk's gates into LDS with 16-byte loads, all
        // issued before any store (rows past the chunk end read as zero)
        {
            constexpr int GV = BT * DK / 4 / 256;    // vectors per thread
            f32x4 gv[GV];
#pragma unroll
            for (int i = 0; i < GV; ++i) {
                const int e4 = tid + 256 * i, r = e4 / (DK / 4), c4 = (e4 % (DK / 4)) * 4;
                gv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (r < len) gv[i] = *reinterpret_cast<const f32x4*>(a.g + ((t0 + r) * H + head) * DK + c4);
            }
#pragma unroll
            for (int i = 0; i < GV; ++i) {
                const int e4 = tid + 256 * i, r = e4 / (DK / 4), c4 = (e4 % (DK / 4)) * 4;
                *reinterpret_cast<f32x4*>(&Gs[r * (DK + 4) + c4]) = gv[i];
            }
        }
        __syncthreads();
        // running sum down each key column, in fp64 so that every G is the
        // correctly rounded prefix sum (rows past the end keep the last sum):
        // lane l of wave w sums key 32w + (l & 31) over rows 32 (l >> 5) ..
        // +31 in order, the upper half starting from the lower half's total
        {
            const int d = 32 * w + (lane & 31), r0 = 32 * (lane >> 5);
            float gv[32];
#pragma unroll
            for (int r = 0; r < 32; ++r) gv[r] = Gs[(r0 + r) * (DK + 4) + d];
            double half = 0.0;
#pragma unroll
            for (int r = 0; r < 32; ++r) half += (double)gv[r];
            const double lo = __shfl(half, lane & 31, 64);
            double xs = lane >= 32 ? lo : 0.0;
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                xs += (double)gv[r];
                const float x = (float)xs;
                Gs[(r0 + r) * (DK + 4) + d] = x;
                if (a.g_cumsum && r0 + r < len) a.g_cumsum[((t0 + r0 + r) * H + head) * DK + d] = x;
            }
            if (lane >= 32) a.ws.gamL[ch * DK + d] = (float)xs;
        }
    }
    __syncthreads();

    // ---- L = strictly lower (beta_i k_i.k_j b^{G_i-G_j}) on MFMA, 10 tiles over 4 waves.
    // Per key, an off-diagonal tile (I > J) factors the decay about the last
    // row of block J, so that both factors are at most 1 for any g <= 0; a
    // diagonal tile does the same when its block's gate range allows (below),
    // and takes the exponent differences directly otherwise.
    // four rows i0 .. i0+3 against row j: sum_d x_id k_jd b^{G_id - G_jd},
    // 16-byte reads of four keys at a time, row j's k and G shared by the rows
    auto direct4 = [&](const Op* xi, int i0, int j, float* out) {
        float s[4] = {0.f, 0.f, 0.f, 0.f};
        for (int d = 0; d < DK; d += 4) {
            const f32x4 kj = *reinterpret_cast<const f32x4*>(&kt[j * LDQ + d]);
            const f32x4 gj = *reinterpret_cast<const f32x4*>(&Gs[j * (DK + 4) + d]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 xv = *reinterpret_cast<const f32x4*>(&xi[(i0 + r) * LDQ + d]);
                const f32x4 gi = *reinterpret_cast<const f32x4*>(&Gs[(i0 + r) * (DK + 4) + d]);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[r] += xv[e] * kj[e] * fpow(gi[e] - gj[e], a.use_exp2);
            }
        }
        for (int r = 0; r < 4; ++r) out[r] = s[r];
    };
    // eight consecutive fp32 values of an LDS row (16-byte aligned) into registers
    auto ld8 = [](const float* p, float* x) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(p), w2 = *reinterpret_cast<const f32x4*>(p + 4);
        for (int e = 0; e < 4; ++e) { x[e] = u[e]; x[e + 4] = w2[e]; }
    };
    // row i against the four rows j0 .. j0+3: sum_d x_id k_jd b^{G_id - G_jd}
    auto direct4j = [&](const Op* xi, int i, int j0, float* out) {
        float s[4] = {0.f, 0.f, 0.f, 0.f};
        for (int d = 0; d < DK; d += 4) {
            const f32x4 xv = *reinterpret_cast<const f32x4*>(&xi[i * LDQ + d]);
            const f32x4 gi = *reinterpret_cast<const f32x4*>(&Gs[i * (DK + 4) + d]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 kj = *reinterpret_cast<const f32x4*>(&kt[(j0 + r) * LDQ + d]);
                const f32x4 gj = *reinterpret_cast<const f32x4*>(&Gs[(j0 + r) * (DK + 4) + d]);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[r] += xv[e] * kj[e] * fpow(gi[e] - gj[e], a.use_exp2);
            }
        }
        for (int r = 0; r < 4; ++r) out[r] = s[r];
    };
    // A diagonal tile takes the factored form as well when the gate falls by
    // at most 2^8 of decay inside its block on every key: the factor of its
    // rows about the block's last row then stays within 2^8 (the bf16
    // preparation's rule). Wave-uniform.
    auto diag_factored = [&](int blk) {
        float rmax = 0.0f;
        for (int d = lane; d < DK; d += 64)
            rmax = fmaxf(rmax, Gs[(16 * blk) * (DK + 4) + d] - Gs[(16 * blk + 15) * (DK + 4) + d]);
        return __all(rmax <= (a.use_exp2 ? 8.0f : 5.545177444479562f)) != 0;
    };
    for (int t = w; t < 10; t += 4) {
        const int it = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        const int jt = t - (it * (it + 1)) / 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (PERKEY && it == jt && !diag_factored(it)) {
            // lanes whose column is past all four rows skip the sums
            float dv[4] = {0.f, 0.f, 0.f, 0.f};
            const int i0 = 16 * it + 4 * G, j = 16 * jt + n;
            if (j < i0 + 3) direct4(kt, i0, j, dv);
            for (int r = 0; r < 4; ++r) acc[r] = j < i0 + r ? dv[r] : 0.0f;
        } else {
            for (int kk = 0; kk < DK / 32; ++kk) {
                const int col = 32 * kk + 8 * G;
                if (!PERKEY) {
                    P::mma(acc, P::ld(&kt[(16 * it + n) * LDQ + col]), P::ld(&kt[(16 * jt + n) * LDQ + col]));
                } else {
                    const int ref = 16 * jt + 15;
                    float gr[8], gi[8], gj[8], ki[8], kj[8], xa[8], xb[8];
                    ld8(&Gs[ref * (DK + 4) + col], gr);
                    ld8(&Gs[(16 * it + n) * (DK + 4) + col], gi);
                    ld8(&Gs[(16 * jt + n) * (DK + 4) + col], gj);
                    ld8(&kt[(16 * it + n) * LDQ + col], ki);
                    ld8(&kt[(16 * jt + n) * LDQ + col], kj);
                    for (int e = 0; e < 8; ++e) {
                        xa[e] = ki[e] * fpow(gi[e] - gr[e], a.use_exp2);
                        xb[e] = kj[e] * fpow(gr[e] - gj[e], a.use_exp2);
                    }
                    P::mma(acc, P::from(xa), P::from(xb));
                }
            }
        }
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * it + 4 * G + r, j = 16 * jt + n;
            float l = 0.0f;
            if (j < i) {
                l = bet[i] * acc[r];
                if (!PERKEY) l *= fpow(Gs[i] - Gs[j], a.use_exp2);
            }
            Ls[i * LDL + j] = l;
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

    // ---- T out as operands (row-major 64 x 64), optional token-major fp32 A slot
    Op* Tw = reinterpret_cast<Op*>(a.ws.Tm) + ch * (BT * BT);
    for (int e = tid; e < BT * BT / 4; e += 256) {
        const int r = e / (BT / 4), c4 = (e % (BT / 4)) * 4;
        f32x4 x;
        for (int q2 = 0; q2 < 4; ++q2) x[q2] = Ts[r * LDL + c4 + q2];
        P::f32_to_op4(Tw + r * BT + c4, x);
        if (a.A && r < len) *reinterpret_cast<f32x4*>(a.A + ((t0 + r) * H + head) * BT + c4) = x;
    }

    // ---- P = tril_incl(q k^T decayed) as operands, computed as P^T tiles
    // (rows j of block jt, columns i of block it); blocks above the diagonal
    // are written as zeros
    if (has_q) {
        Op* Pw = reinterpret_cast<Op*>(a.ws.P) + ch * (BT * BT);
        for (int t = w; t < 16; t += 4) {
            const int jt = t >> 2, it = t & 3;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (PERKEY && jt == it && !diag_factored(jt)) {
                float dv[4] = {0.f, 0.f, 0.f, 0.f};
                const int i = 16 * it + n, j0 = 16 * jt + 4 * G;
                if (j0 <= i) direct4j(qt, i, j0, dv);
                for (int r = 0; r < 4; ++r) acc[r] = j0 + r <= i ? dv[r] : 0.0f;
            } else if (jt <= it) {
                for (int kk = 0; kk < DK / 32; ++kk) {
                    const int col = 32 * kk + 8 * G;
                    if (!PERKEY) {
                        P::mma(acc, P::ld(&kt[(16 * jt + n) * LDQ + col]), P::ld(&qt[(16 * it + n) * LDQ + col]));
                    } else {
                        const int ref = 16 * jt + 15;
                        float gr[8], gi[8], gj[8], kj[8], qi[8], xa[8], xb[8];
                        ld8(&Gs[ref * (DK + 4) + col], gr);
                        ld8(&Gs[(16 * it + n) * (DK + 4) + col], gi);
                        ld8(&Gs[(16 * jt + n) * (DK + 4) + col], gj);
                        ld8(&kt[(16 * jt + n) * LDQ + col], kj);
                        ld8(&qt[(16 * it + n) * LDQ + col], qi);
                        for (int e = 0; e < 8; ++e) {
                            xa[e] = kj[e] * fpow(gr[e] - gj[e], a.use_exp2);
                            xb[e] = qi[e] * fpow(gi[e] - gr[e], a.use_exp2);
                        }
                        P::mma(acc, P::from(xa), P::from(xb));
                    }
                }
            }
            const int i = 16 * it + n;
            float x[4];
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jt + 4 * G + r;
                float pv = j <= i ? acc[r] : 0.0f;
                if (!PERKEY && j <= i) pv *= fpow(Gs[i] - Gs[j], a.use_exp2);
                x[r] = pv;
            }
            P::st4(Pw + i * BT + 16 * jt + 4 * G, x);
        }
    }

    if (PERKEY) {
        // gated q and k tiles as operands: q*b^G, k*b^G, k*b^{G_last-G}
        Op* qg = reinterpret_cast<Op*>(a.ws.qg) + ch * (BT * DK);
        Op* kd = reinterpret_cast<Op*>(a.ws.kd) + ch * (BT * DK);
        Op* kg = reinterpret_cast<Op*>(a.ws.kg) + ch * (BT * DK);
        const int last = len > 0 ? len - 1 : 0;
        for (int e4 = tid; e4 < BT * DK / 4; e4 += 256) {
            const int r = e4 / (DK / 4), c4 = (e4 % (DK / 4)) * 4;
            float xq[4], xd[4], xg[4];
            const f32x4 gg = *reinterpret_cast<const f32x4*>(&Gs[r * (DK + 4) + c4]);
            const f32x4 gl = *reinterpret_cast<const f32x4*>(&Gs[last * (DK + 4) + c4]);
            const f32x4 kv = *reinterpret_cast<const f32x4*>(&kt[r * LDQ + c4]);
            const f32x4 qv = *reinterpret_cast<const f32x4*>(&qt[r * LDQ + c4]);
            for (int e = 0; e < 4; ++e) {
                const float bg = fpow(gg[e], a.use_exp2);
                xq[e] = qv[e] * bg;
                xd[e] = kv[e] * bg;
                xg[e] = kv[e] * fpow(gl[e] - gg[e], a.use_exp2);
            }
            const int cp = c4;
            if (has_q) P::st4(qg + r * DK + cp, xq);
            P::st4(kd + r * DK + cp, xd);
            P::st4(kg + r * DK + cp, xg);
        }
    }
}

// ------------------------------------------------------------------ prep, per-key gate, backward (bf16 in)
// The backward's fp32 preparation for bf16 inputs with a per-key gate: the
// same T, P, gated tiles and G_last as prep_kernel<PolicyF, true> would give
// for the widened inputs, with its steps reordered so that two workgroups
// share a compute unit (67 KiB of LDS). k and q stay bf16 in LDS (they widen
// to fp32 exactly at every read); the L tiles wait in registers while P and
// the gated tiles are formed, and the inverse then runs over the dead k, q
// and gate tiles. No input transforms (the backward takes the transformed
// inputs).
constexpr int KQB = DK + 8;     // bf16 row stride of the k and q tiles (272 bytes)
constexpr int GSL = DK + 4;     // fp32 row stride of the gate tile

// 8 bf16 (16 bytes) -> fp32
__device__ __forceinline__ void bf8_to_f32(const bf16* p, float* x) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, v[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, v[i] & 0xffff0000u);
    }
}
// 4 bf16 (8 bytes) -> fp32
__device__ __forceinline__ f32x4 bf4_to_f32(const bf16* p) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    return f32x4{__builtin_bit_cast(float, v[0] << 16), __builtin_bit_cast(float, v[0] & 0xffff0000u),
                 __builtin_bit_cast(float, v[1] << 16), __builtin_bit_cast(float, v[1] & 0xffff0000u)};
}

__global__ __launch_bounds__(256, 2) void prep_kernel_pkb(PrepArgs a) {
    constexpr int KQ_BYTES = 2 * BT * KQB * 2, G_BYTES = BT * GSL * 4;
    __shared__ __attribute__((aligned(16))) char smem[KQ_BYTES + G_BYTES];
    __shared__ float bet[BT];
    bf16* kt = reinterpret_cast<bf16*>(smem);
    bf16* qt = kt + BT * KQB;
    float* Gs = reinterpret_cast<float*>(smem + KQ_BYTES);
    // once P and the gated tiles are out: L, T and the inverse's scratch
    float* Ls = reinterpret_cast<float*>(smem);
    float* Ts = Ls + BT * LDL;
    float* Yb = Ts + BT * LDL;
    static_assert((2 * BT * LDL + 3 * 16 * 17) * 4 <= KQ_BYTES + G_BYTES, "L, T and scratch fit the tiles");

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, G = lane >> 4, n = lane & 15;
    const int ci = blockIdx.x, head = blockIdx.y, H = a.H;
    int u, cc;
    chunk_of(a.um, ci, u, cc);
    if (u < 0) return;
    const UnitInfo ui = unit_info(a.um, u);
    const int64_t t0 = ui.start + (int64_t)cc * BT;
    int len = ui.len - cc * BT;
    len = len < 0 ? 0 : (len > BT ? BT : len);
    const int64_t ch = (int64_t)ci * H + head;
    const bf16* kin = reinterpret_cast<const bf16*>(a.k);
    const bf16* qin = reinterpret_cast<const bf16*>(a.q);

    // ---- every load issued before any store (rows past the chunk end are zero)
    {
        u32x4 kv[4], qv[4];
        f32x4 gv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i, r = e >> 4, c8 = (e & 15) * 8;
            kv[i] = u32x4{0u, 0u, 0u, 0u};
            qv[i] = kv[i];
            if (r < len) {
                kv[i] = *reinterpret_cast<const u32x4*>(kin + ((t0 + r) * H + head) * DK + c8);
                qv[i] = *reinterpret_cast<const u32x4*>(qin + ((t0 + r) * H + head) * DK + c8);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e4 = tid + 256 * i, r = e4 >> 5, c4 = (e4 & 31) * 4;
            gv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (r < len) gv[i] = *reinterpret_cast<const f32x4*>(a.g + ((t0 + r) * H + head) * DK + c4);
        }
        const float bt = tid < len ? (float)reinterpret_cast<const bf16*>(a.beta)[(t0 + tid) * H + head] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i, r = e >> 4, c8 = (e & 15) * 8;
            *reinterpret_cast<u32x4*>(kt + r * KQB + c8) = kv[i];
            *reinterpret_cast<u32x4*>(qt + r * KQB + c8) = qv[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e4 = tid + 256 * i, r = e4 >> 5, c4 = (e4 & 31) * 4;
            *reinterpret_cast<f32x4*>(&Gs[r * GSL + c4]) = gv[i];
        }
        if (tid < BT) bet[tid] = bt;
    }
    __syncthreads();
    // ---- running sum down each key column in fp64 (the correctly rounded
    // prefix sums): lane l of wave w sums key 32w + (l & 31) over rows
    // 32 (l >> 5) .. +31 in order, the upper half from the lower half's total
    {
        const int d = 32 * w + (lane & 31), r0 = 32 * (lane >> 5);
        float gv[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) gv[r] = Gs[(r0 + r) * GSL + d];
        double half = 0.0;
#pragma unroll
        for (int r = 0; r < 32; ++r) half += (double)gv[r];
        const double lo = __shfl(half, lane & 31, 64);
        double xs = lane >= 32 ? lo : 0.0;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            xs += (double)gv[r];
            Gs[(r0 + r) * GSL + d] = (float)xs;
        }
        if (lane >= 32) a.ws.gamL[ch * DK + d] = (float)xs;
    }
    __syncthreads();

    // four rows i0 .. i0+3 against row j (i0 + r > j): sum_d x_id k_jd b^{G_id - G_jd}
    auto direct4 = [&](const bf16* xi, int i0, int j, float* out) {
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int d = 0; d < DK; d += 4) {
            const f32x4 kj = bf4_to_f32(kt + j * KQB + d);
            const f32x4 gj = *reinterpret_cast<const f32x4*>(&Gs[j * GSL + d]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 xv = bf4_to_f32(xi + (i0 + r) * KQB + d);
                const f32x4 gi = *reinterpret_cast<const f32x4*>(&Gs[(i0 + r) * GSL + d]);
#pragma unroll
                for (int e = 0; e < 4; ++e) s4[r] += xv[e] * kj[e] * fpow(gi[e] - gj[e], a.use_exp2);
            }
        }
        for (int r = 0; r < 4; ++r) out[r] = s4[r];
    };
    // row i against the four rows j0 .. j0+3
    auto direct4j = [&](const bf16* xi, int i, int j0, float* out) {
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int d = 0; d < DK; d += 4) {
            const f32x4 xv = bf4_to_f32(xi + i * KQB + d);
            const f32x4 gi = *reinterpret_cast<const f32x4*>(&Gs[i * GSL + d]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 kj = bf4_to_f32(kt + (j0 + r) * KQB + d);
                const f32x4 gj = *reinterpret_cast<const f32x4*>(&Gs[(j0 + r) * GSL + d]);
#pragma unroll
                for (int e = 0; e < 4; ++e) s4[r] += xv[e] * kj[e] * fpow(gi[e] - gj[e], a.use_exp2);
            }
        }
        for (int r = 0; r < 4; ++r) out[r] = s4[r];
    };
    auto ld8 = [](const float* p, float* x) {
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(p), u1 = *reinterpret_cast<const f32x4*>(p + 4);
        for (int e = 0; e < 4; ++e) { x[e] = u0[e]; x[e + 4] = u1[e]; }
    };
    // the factored form for a diagonal tile too when the gate falls by at
    // most 2^8 of decay inside its block on every key (wave-uniform)
    auto diag_factored = [&](int blk) {
        float rmax = 0.0f;
        for (int d = lane; d < DK; d += 64) rmax = fmaxf(rmax, Gs[(16 * blk) * GSL + d] - Gs[(16 * blk + 15) * GSL + d]);
        return __all(rmax <= (a.use_exp2 ? 8.0f : 5.545177444479562f)) != 0;
    };
    // the 16 x 16 tile of sum_d x_id k_jd b^{G_id - G_jd} for rows i = 16 it + .
    // of x and j = 16 jt + . of k, with the decay factored about the last row
    // of block jt: x b^{G_i - G_ref} and k b^{G_ref - G_j}, both at most |x|,
    // |k| off the diagonal. Lane holds (i = 16 it + 4G + r, j = 16 jt + n), or
    // transposed (j = 16 jt + 4G + r, i = 16 it + n).
    auto factored = [&](const bf16* x_t, int it, int jt, bool transposed) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int ref = 16 * jt + 15, i = 16 * it + n, j = 16 * jt + n;
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const int col = 32 * kk + 8 * G;
            float gr[8], gi[8], gj[8], xi[8], kj[8];
            ld8(&Gs[ref * GSL + col], gr);
            ld8(&Gs[i * GSL + col], gi);
            ld8(&Gs[j * GSL + col], gj);
            bf8_to_f32(x_t + i * KQB + col, xi);
            bf8_to_f32(kt + j * KQB + col, kj);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float fi = xi[e] * fpow(gi[e] - gr[e], a.use_exp2), fj = kj[e] * fpow(gr[e] - gj[e], a.use_exp2);
                acc = transposed ? __builtin_amdgcn_mfma_f32_16x16x4f32(fj, fi, acc, 0, 0, 0)
                                 : __builtin_amdgcn_mfma_f32_16x16x4f32(fi, fj, acc, 0, 0, 0);
            }
        }
        return acc;
    };

    // ---- L = strictly lower (beta_i k_i.k_j b^{G_i - G_j}), 10 tiles over
    // 4 waves, kept in registers (tile w + 4q; lane holds L[16it + 4G + r][16jt + n])
    f32x4 lacc[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        lacc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int t = w + 4 * q;
        if (t >= 10) continue;
        const int it = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        const int jt = t - (it * (it + 1)) / 2;
        f32x4 acc;
        if (it == jt && !diag_factored(it)) {
            float dv[4] = {0.f, 0.f, 0.f, 0.f};
            const int i0 = 16 * it + 4 * G, j = 16 * jt + n;
            if (j < i0 + 3) direct4(kt, i0, j, dv);
            for (int r = 0; r < 4; ++r) acc[r] = j < i0 + r ? dv[r] : 0.0f;
        } else {
            acc = factored(kt, it, jt, false);
        }
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * it + 4 * G + r, j = 16 * jt + n;
            lacc[q][r] = j < i ? bet[i] * acc[r] : 0.0f;
        }
    }

    // ---- P = tril_incl(q k^T decayed), computed as P^T tiles (rows j of
    // block jt, columns i of block it); blocks above the diagonal are zeros
    {
        float* Pw = reinterpret_cast<float*>(a.ws.P) + ch * (BT * BT);
        for (int t = w; t < 16; t += 4) {
            const int jt = t >> 2, it = t & 3;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (jt == it && !diag_factored(jt)) {
                float dv[4] = {0.f, 0.f, 0.f, 0.f};
                const int i = 16 * it + n, j0 = 16 * jt + 4 * G;
                if (j0 <= i) direct4j(qt, i, j0, dv);
                for (int r = 0; r < 4; ++r) acc[r] = j0 + r <= i ? dv[r] : 0.0f;
            } else if (jt <= it) {
                acc = factored(qt, it, jt, true);
            }
            const int i = 16 * it + n;
            f32x4 x;
            for (int r = 0; r < 4; ++r) x[r] = 16 * jt + 4 * G + r <= i ? acc[r] : 0.0f;
            *reinterpret_cast<f32x4*>(Pw + i * BT + 16 * jt + 4 * G) = x;
        }
    }

    // ---- gated q and k tiles: q b^G, k b^G, k b^{G_last - G}
    {
        float* qg = reinterpret_cast<float*>(a.ws.qg) + ch * (BT * DK);
        float* kd = reinterpret_cast<float*>(a.ws.kd) + ch * (BT * DK);
        float* kg = reinterpret_cast<float*>(a.ws.kg) + ch * (BT * DK);
        const int last = len > 0 ? len - 1 : 0;
        for (int e4 = tid; e4 < BT * DK / 4; e4 += 256) {
            const int r = e4 / (DK / 4), c4 = (e4 % (DK / 4)) * 4;
            const f32x4 gg = *reinterpret_cast<const f32x4*>(&Gs[r * GSL + c4]);
            const f32x4 gl = *reinterpret_cast<const f32x4*>(&Gs[last * GSL + c4]);
            const f32x4 kv = bf4_to_f32(kt + r * KQB + c4), qv = bf4_to_f32(qt + r * KQB + c4);
            f32x4 xq, xd, xg;
            for (int e = 0; e < 4; ++e) {
                const float bg = fpow(gg[e], a.use_exp2);
                xq[e] = qv[e] * bg;
                xd[e] = kv[e] * bg;
                xg[e] = kv[e] * fpow(gl[e] - gg[e], a.use_exp2);
            }
            *reinterpret_cast<f32x4*>(qg + r * DK + c4) = xq;
            *reinterpret_cast<f32x4*>(kd + r * DK + c4) = xd;
            *reinterpret_cast<f32x4*>(kg + r * DK + c4) = xg;
        }
    }
    __syncthreads();                             // k, q and G are dead from here
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const int t = w + 4 * q;
        if (t >= 10) continue;
        const int it = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        const int jt = t - (it * (it + 1)) / 2;
        for (int r = 0; r < 4; ++r) Ls[(16 * it + 4 * G + r) * LDL + 16 * jt + n] = lacc[q][r];
    }
    __syncthreads();

    // ---- T = (I + L)^{-1}: 16 x 16 diagonal blocks by substitution (wave 0,
    // lane = block * 16 + column), then the off-diagonal blocks by distance
    if (w == 0) {
        const int bk = lane >> 4, c = lane & 15, o = 16 * bk;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float sacc = 0.0f;
#pragma unroll
            for (int j = 0; j < i; ++j) sacc += Ls[(o + i) * LDL + o + j] * x[j];
            x[i] = i == c ? 1.0f : (i > c ? -sacc : 0.0f);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Ts[(o + i) * LDL + o + c] = x[i];
    } else {
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
            float sacc = 0.0f;
            for (int K2 = J; K2 < I; ++K2)
                for (int m = 0; m < 16; ++m)
                    sacc += Ls[(16 * I + rr) * LDL + 16 * K2 + m] * Ts[(16 * K2 + m) * LDL + 16 * J + cc2];
            Yb[(bi * 16 + rr) * 17 + cc2] = sacc;
        }
        __syncthreads();
        for (int e = tid; e < nb * 256; e += 256) {
            const int bi = e >> 8, rr = (e >> 4) & 15, cc2 = e & 15;
            const int I = d + bi, J = bi;
            float sacc = 0.0f;
            for (int m = 0; m < 16; ++m) sacc += Ts[(16 * I + rr) * LDL + 16 * I + m] * Yb[(bi * 16 + m) * 17 + cc2];
            Ts[(16 * I + rr) * LDL + 16 * J + cc2] = -sacc;
        }
        __syncthreads();
    }
    float* Tw = reinterpret_cast<float*>(a.ws.Tm) + ch * (BT * BT);
    for (int e = tid; e < BT * BT / 4; e += 256) {
        const int r = e / (BT / 4), c4 = (e % (BT / 4)) * 4;
        f32x4 x;
        for (int q2 = 0; q2 < 4; ++q2) x[q2] = Ts[r * LDL + c4 + q2];
        *reinterpret_cast<f32x4*>(Tw + r * BT + c4) = x;
    }
}

// ------------------------------------------------------------------ prep, fp16 scalar gate
// One wave per (chunk, head) with every tile in registers. Fragment (b, kk)
// of a 64 x 128 input tile: lane (G, n) holds elements 32kk + 8G .. +7 of row
// 16b + n (the 16x16x32 fp16 MFMA operand layout). With k_K as A and k_I (or
// q_I) as B the product over the 128 keys leaves lane (G, n) holding the
// value for token i = 16I + n against token j = 16K + 4G + r: block (I, K) of
// k k^T (of q k^T) in "row layout" R(X), lane holding X[n][4G .. 4G+3]. The
// accumulator layout C(X) holds X[4G .. 4G+3][n]. With 16x16x4 fp32 MFMAs
// contracting over k = 4G + s (s = 0..3)
//     mm4(R(A), C(B)) = C(AB),   mm4(C(B), R(A)) = R(AB),
// so the blockwise inverse of (I + L) chains on MFMA with no lane exchange:
// diagonal 16 x 16 blocks T_II by forward substitution (lane = block, column;
// rows through LDS), then T_IJ = -T_II sum_{J<=K<I} L_IK T_KJ by distance.
// The state pass reads T and P (fp16, op_pos columns) and the coefficient
// block from here; it converts k and q itself.
__device__ __forceinline__ f32x4 mm4(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
    return c;
}

// 8 bf16 (16 bytes) -> the same 8 values as fp16 (exact in the fp16 normal range)
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __builtin_bit_cast(float, w[i] << 16), hi = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        o[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
    return o;
}

// 4 fp32 -> 4 fp16, rounded to nearest
__device__ __forceinline__ u32x2 f32x4_to_f16x4(f32x4 x) {
    f16x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (f16)x[e];
    return __builtin_bit_cast(u32x2, h);
}

constexpr int PLS = 20;               // row stride (floats) of the 16 x 16 LDS blocks
constexpr int PBL = 16 * PLS + 4;     // L blocks: successive blocks 4 banks apart
constexpr int PBT = 16 * PLS + 16;    // T blocks: successive blocks 16 banks apart

// XF: the input transforms or their slots are asked for (a separate
// instantiation, so that the plain preparation keeps its registers).
// BWD: the preparation the backward reads instead: T itself and P as fp16 in
// natural order (every block, zeros above the diagonal) and the fp32 gate
// rows G, b^G, b^{G_L - G}, b^{G_L}, b^G (no input transforms).
template <bool XF, bool BWD = false>
__global__ __launch_bounds__(64) void prep_kernel_h(PrepArgs a) {
    __shared__ __attribute__((aligned(16))) float Ld[4 * PBL];
    __shared__ __attribute__((aligned(16))) float Td[4 * PBT];
    __shared__ __attribute__((aligned(16))) float Gs[BT];
    __shared__ __attribute__((aligned(16))) float Bs[BT];
    __shared__ __attribute__((aligned(16))) float Rk[BT];
    __shared__ __attribute__((aligned(16))) float Rq[BT];

    // heads vary fastest across the grid, so that waves dispatched together
    // read the same token rows (all heads of a row are contiguous)
    const int lane = threadIdx.x, G = lane >> 4, n = lane & 15;
    const int H = a.H, ci = (int)(blockIdx.x / (uint32_t)H), head = (int)(blockIdx.x - (uint32_t)ci * H);
    int u, cc;
    chunk_of(a.um, ci, u, cc);
    u = __builtin_amdgcn_readfirstlane(u);
    cc = __builtin_amdgcn_readfirstlane(cc);
    if (u < 0) return;
    const UnitInfo ui = uniform(unit_info(a.um, u));
    const int64_t t0 = ui.start + (int64_t)cc * BT;
    int len = ui.len - cc * BT;
    len = len < 0 ? 0 : (len > BT ? BT : len);
    const int64_t ch = (int64_t)ci * H + head;
    const bool has_q = a.q != nullptr;

    // ---- every load up front; buffer ranges end at the chunk's last token,
    // so rows past it read as zero
    const uint32_t rowb = (uint32_t)H * DK * 2;   // bytes between token rows of k and q
    const int64_t e0 = t0 * H + head;             // element index of token t0 in the gate arrays
    const uint32_t span16 = len > 0 ? (uint32_t)(len - 1) * rowb + DK * 2 : 0;
    const rsrc_t rg = make_rsrc(a.g + e0, len > 0 ? ((uint32_t)(len - 1) * H + 1) * 4 : 0);
    const rsrc_t rb = make_rsrc(reinterpret_cast<const bf16*>(a.beta) + e0, len > 0 ? ((uint32_t)(len - 1) * H + 1) * 2 : 0);
    const rsrc_t rk = make_rsrc(reinterpret_cast<const bf16*>(a.k) + e0 * DK, span16);
    const rsrc_t rq = make_rsrc(has_q ? reinterpret_cast<const bf16*>(a.q) + e0 * DK : a.k, has_q ? span16 : 0);
    const float gv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, lane * H * 4, 0, 0));
    const uint32_t braw = __builtin_amdgcn_raw_buffer_load_b16(rb, lane * H * 2, 0, 0);
    u32x4 kf[4][4], qf[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            kf[b][kk] = __builtin_amdgcn_raw_buffer_load_b128(rk, (16 * b + n) * rowb + (32 * kk + 8 * G) * 2, 0, 0);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qf[b][kk] = __builtin_amdgcn_raw_buffer_load_b128(rq, (16 * b + n) * rowb + (32 * kk + 8 * G) * 2, 0, 0);

    // ---- input transforms: the reciprocal norms r of the k and q rows (the
    // four lanes of a row, G = 0..3, sum their 32 keys and exchange by xor)
    // and beta through a sigmoid; optional slots of the transformed inputs
    float rkb[4] = {1.f, 1.f, 1.f, 1.f}, rqb[4] = {1.f, 1.f, 1.f, 1.f};
    if (XF && a.qk_norm) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float sk = 0.0f, sq = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float k0 = __builtin_bit_cast(float, kf[b][kk][i] << 16), k1 = __builtin_bit_cast(float, kf[b][kk][i] & 0xffff0000u);
                    const float q0 = __builtin_bit_cast(float, qf[b][kk][i] << 16), q1 = __builtin_bit_cast(float, qf[b][kk][i] & 0xffff0000u);
                    sk += k0 * k0 + k1 * k1;
                    sq += q0 * q0 + q1 * q1;
                }
            sk += __shfl_xor(sk, 16, 64);
            sk += __shfl_xor(sk, 32, 64);
            sq += __shfl_xor(sq, 16, 64);
            sq += __shfl_xor(sq, 32, 64);
            // rows past the chunk end (zero) keep r = 1
            rkb[b] = 16 * b + n < len ? rnorm_f(sk) : 1.0f;
            rqb[b] = 16 * b + n < len ? rnorm_f(sq) : 1.0f;
        }
    }
    if (G == 0)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            Rk[16 * b + n] = rkb[b];
            Rq[16 * b + n] = rqb[b];
        }
    if (XF && (a.k_hat || (has_q && a.q_hat))) {
        // x r rounded to bf16, at the positions the fragments were loaded from
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (16 * b + n >= len) continue;
            const int64_t rowe = (e0 + (int64_t)(16 * b + n) * H) * DK;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                u32x4 wk, wq;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    auto rb = [](uint32_t w, float r) {
                        const float lo = __builtin_bit_cast(float, w << 16) * r, hi = __builtin_bit_cast(float, w & 0xffff0000u) * r;
                        return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)hi) << 16);
                    };
                    wk[i] = rb(kf[b][kk][i], rkb[b]);
                    wq[i] = rb(qf[b][kk][i], rqb[b]);
                }
                if (a.k_hat) *reinterpret_cast<u32x4*>(reinterpret_cast<bf16*>(a.k_hat) + rowe + 32 * kk + 8 * G) = wk;
                if (has_q && a.q_hat) *reinterpret_cast<u32x4*>(reinterpret_cast<bf16*>(a.q_hat) + rowe + 32 * kk + 8 * G) = wq;
            }
        }
    }

    // ---- inclusive scan of the gate (lane = token; zero past the chunk end)
    float x = gv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    const float xl = __shfl(x, len > 0 ? len - 1 : 0, 64);
    float bt = __builtin_bit_cast(float, braw << 16);
    if (XF && a.beta_sig) bt = lane < len ? sigmoid_f(bt) : 0.0f;
    Gs[lane] = x;
    Bs[lane] = bt;
    __syncthreads();   // Rk, Rq
    {
        const float bG = fpow(x, a.use_exp2), bLG = fpow(xl - x, a.use_exp2);
        const float rk = XF ? Rk[lane] : 1.0f, rq = XF ? Rq[lane] : 1.0f;
        if (BWD) {
            float* gw = a.ws.gam + ch * (GAMR * BT);
            gw[lane] = x;
            gw[BT + lane] = bG;
            gw[2 * BT + lane] = bLG;
            gw[3 * BT + lane] = fpow(xl, a.use_exp2);
            gw[4 * BT + lane] = bG;
        } else {
            float* cf = reinterpret_cast<float*>(a.ws.cfh) + ch * (CFS / 4);
            const int lo = lane_order(lane);
            cf[CS_CP + lo] = bLG * rk;
            cf[CS_BG + lo] = bG * rk;
            cf[CS_BQ + lo] = bG * rq;
            if (lane == 0) cf[CS_EL] = fpow(xl, a.use_exp2);
        }
        if (a.g_cumsum && lane < len) a.g_cumsum[e0 + (int64_t)lane * H] = x;
        if (XF && lane < len) {
            if (a.k_rstd) a.k_rstd[e0 + (int64_t)lane * H] = rk;
            if (has_q && a.q_rstd) a.q_rstd[e0 + (int64_t)lane * H] = rq;
            if (a.beta_eff) reinterpret_cast<bf16*>(a.beta_eff)[e0 + (int64_t)lane * H] = (bf16)bt;
        }
    }
    float Gi[4], Bi[4];
    f32x4 Gj[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        Gi[b] = Gs[16 * b + n];
        Bi[b] = Bs[16 * b + n];
        Gj[b] = *reinterpret_cast<const f32x4*>(&Gs[16 * b + 4 * G]);
    }

    // ---- k and q as fp16 operands
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            kf[b][kk] = bf16x8_to_f16x8(kf[b][kk]);
            qf[b][kk] = bf16x8_to_f16x8(qf[b][kk]);
        }

    // ---- Gram and q k^T blocks (I, K), K <= I: decay, P out, L kept
    f16* Pw = reinterpret_cast<f16*>(a.ws.P) + ch * (BT * BT);
    f32x4 TL[4][4];   // R(L_IK), K < I
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
        for (int K = 0; K < 4; ++K) {
            f16* pdst = Pw + (16 * I + n) * BT + (BWD ? 16 * K + 4 * G : op_pos(16 * K + 4 * G));
            if (K > I) {
                // zero blocks; rows 0..31 of the state pass read columns 0..31 only
                if (BWD || (has_q && (I >= 2 || K < 2))) *reinterpret_cast<u32x2*>(pdst) = u32x2{0u, 0u};
                continue;
            }
            f32x4 gk = {0.f, 0.f, 0.f, 0.f}, gq = gk;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const f16x8 A = __builtin_bit_cast(f16x8, kf[K][kk]);
                gk = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(f16x8, kf[I][kk]), gk, 0, 0, 0);
                if (has_q) gq = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(f16x8, qf[I][kk]), gq, 0, 0, 0);
            }
            f32x4 pv, lv;
            const f32x4 rkj = XF ? *reinterpret_cast<const f32x4*>(&Rk[16 * K + 4 * G]) : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool le = K < I || 4 * G + r <= n, lt = K < I || 4 * G + r < n;
                const float d = le ? fpow(Gi[I] - Gj[K][r], a.use_exp2) * rkj[r] : 0.0f;
                pv[r] = le ? gq[r] * d * rqb[I] : 0.0f;
                lv[r] = lt ? Bi[I] * gk[r] * d * rkb[I] : 0.0f;
            }
            if (has_q) *reinterpret_cast<u32x2*>(pdst) = f32x4_to_f16x4(pv);
            if (K < I) TL[I][K] = lv;
            else *reinterpret_cast<f32x4*>(&Ld[I * PBL + n * PLS + 4 * G]) = lv;
        }
    }

    // ---- diagonal blocks: lane (block G, column n) solves (I + L_GG) x = e_n
    {
        const float* Lb = Ld + G * PBL;
        float xs[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int m = 0; 4 * m < i; ++m) {
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lb + i * PLS + 4 * m);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * m + e < i) s += l4[e] * xs[4 * m + e];
            }
            xs[i] = i == n ? 1.0f : (i > n ? -s : 0.0f);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Td[G * PBT + i * PLS + n] = xs[i];
    }
    f32x4 TR[4], TC[3], nTR[4];   // R(T_II), C(T_JJ), R(-T_II)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        TR[b] = *reinterpret_cast<const f32x4*>(&Td[b * PBT + n * PLS + 4 * G]);
        nTR[b] = -TR[b];
        if (b < 3)
#pragma unroll
            for (int r = 0; r < 4; ++r) TC[b][r] = Td[b * PBT + (4 * G + r) * PLS + n];
    }

    // ---- off-diagonal blocks by distance
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 S, R10, R21, R32, R20, R31, R30, C10, C21, C20;
    S = mm4(TL[1][0], TC[0], z4);
    R10 = mm4(S, nTR[1], z4); C10 = mm4(nTR[1], S, z4);
    S = mm4(TL[2][1], TC[1], z4);
    R21 = mm4(S, nTR[2], z4); C21 = mm4(nTR[2], S, z4);
    S = mm4(TL[3][2], TC[2], z4);
    R32 = mm4(S, nTR[3], z4);
    S = mm4(TL[2][1], C10, mm4(TL[2][0], TC[0], z4));
    R20 = mm4(S, nTR[2], z4); C20 = mm4(nTR[2], S, z4);
    S = mm4(TL[3][2], C21, mm4(TL[3][1], TC[1], z4));
    R31 = mm4(S, nTR[3], z4);
    S = mm4(TL[3][2], C20, mm4(TL[3][1], C10, mm4(TL[3][0], TC[0], z4)));
    R30 = mm4(S, nTR[3], z4);

    // ---- T out: T diag(beta) as fp16 operands (op_pos columns) for the state
    // pass, which then needs no beta; the optional token-major fp32 A slot
    // holds T itself
    f16* Tw = reinterpret_cast<f16*>(a.ws.Tm) + ch * (BT * BT);
    const f32x4 TB[4][4] = {{TR[0], z4, z4, z4}, {R10, TR[1], z4, z4}, {R20, R21, TR[2], z4}, {R30, R31, R32, TR[3]}};
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (BWD) {
                *reinterpret_cast<u32x2*>(Tw + (16 * I + n) * BT + 16 * J + 4 * G) = f32x4_to_f16x4(TB[I][J]);
                continue;
            }
            if (I >= 2 || J < 2)   // rows 0..31 of the state pass read columns 0..31 only
                *reinterpret_cast<u32x2*>(Tw + (16 * I + n) * BT + op_pos(16 * J + 4 * G)) =
                    f32x4_to_f16x4(TB[I][J] * *reinterpret_cast<const f32x4*>(&Bs[16 * J + 4 * G]));
            if (a.A && 16 * I + n < len)
                *reinterpret_cast<f32x4*>(a.A + (e0 + (int64_t)(16 * I + n) * H) * BT + 16 * J + 4 * G) = TB[I][J];
        }
}

// ------------------------------------------------------------------ prep, fp16 per-key gate
// One workgroup of four waves per (chunk, head). Wave w owns token rows
// 16w .. 16w+15 (row block w) and lane l the key pair 2l, 2l+1: every load of
// g, k and q is a coalesced 512- or 256-byte row segment, and the per-key
// cumulative gate is a scan in registers plus the column sums of the waves
// before.
//
// The decays of L and P, b^{G_id - G_jd} (j <= i), are factored so that no
// fp16 operand can overflow for any gate g <= 0. With rho_J the gate at the
// last row of block J (rho_{-1} = 0):
//   A side (rows i of block I):  k_i b^{G_i - rho_{I-1}},  q_i b^{G_i - rho_{I-1}}   (<= 1)
//   B side (rows j of block J):  k_j b^{rho_J - G_j}                              (<= 1)
// and tile (I, J) multiplies the B fragment by the per-key factor
// f(I, J) = b^{rho_{I-1} - rho_J}: at most 1 for J < I, and b^{R_I} for the
// diagonal tile, R_I being the block's own gate range. The diagonal tile takes
// this form only when R_I <= PK_DIAG_LOG2 (log2 units) for every key, so that
// the B operand stays within 2^PK_DIAG_LOG2 |k|; otherwise the wave owning
// the block computes its diagonal L and P tiles from direct exponent
// differences in fp32 (VALU), exact for any g <= 0. The state pass's operands
// q b^G, k b^G and k b^{G_L - G} are the A and B forms times per-key factors
// <= 1, so each element costs two exponentials.
//
// L and P are then 16x16x32 MFMA tiles, the inverse runs in LDS over the dead
// operand tiles, and q's A form waits in registers and takes over the first
// operand tile once L is done: 53 KiB of LDS, three workgroups per CU. The
// phases hand data over through LDS only, so their barriers leave the
// workspace stores in flight.
constexpr int PKL = 136;              // row stride (fp16) of the 64 x 128 operand tiles: 272 bytes
constexpr float PK_DIAG_LOG2 = 8.0f;  // largest in-block gate range (log2) of a factored diagonal tile

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float x, float y) {
    f16x2 h;
    h[0] = (f16)x;
    h[1] = (f16)y;
    return __builtin_bit_cast(uint32_t, h);
}

// The tiles (I, J), J <= I, of L and P computed by each wave (its own
// diagonal block first):
//   w0: (0,0) (1,0) (3,2)   w1: (1,1) (2,0)   w2: (2,2) (3,0)   w3: (3,3) (2,1) (3,1)
// and the zero tiles of P (I < J, numbered 0..5) it writes: w0 0, w1 1-2,
// w2 3-4, w3 5.
constexpr int PK_NT[4] = {3, 2, 2, 3};
constexpr int PK_TI[4][3] = {{0, 1, 3}, {1, 2, 0}, {2, 3, 0}, {3, 2, 3}};
constexpr int PK_TJ[4][3] = {{0, 0, 2}, {1, 0, 0}, {2, 0, 0}, {3, 1, 1}};
constexpr int PK_Z0[4] = {0, 1, 3, 5}, PK_NZ[4] = {1, 2, 2, 1};
constexpr int pk_tri(int I, int J) { return I * (I + 1) / 2 + J; }

// Sum over the 64 lanes of 32 per-lane values by recursive halving: at each
// step a lane keeps half of its values and adds the other half received from
// its partner (lanes 32 apart, then 16, 8, 4, 2), so that lanes 2m and 2m+1
// end with the total of value m. The two upper exchanges swap whole 32- and
// 16-lane halves (v_permlane32_swap, v_permlane16_swap); the lower ones move
// one value per lane (row_ror:8, swizzle SWAP 4, quad_perm); the swizzle
// builtin moves ints, so the floats cross it as their bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return u2f(__builtin_amdgcn_update_dpp(0u, f2u(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_sum32(float (&v)[32], int lane) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const auto r = __builtin_amdgcn_permlane32_swap(f2u(v[m]), f2u(v[16 + m]), false, false);
        v[m] = u2f(r[0]) + u2f(r[1]);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const auto r = __builtin_amdgcn_permlane16_swap(f2u(v[m]), f2u(v[8 + m]), false, false);
        v[m] = u2f(r[0]) + u2f(r[1]);
    }
    const bool up8 = lane & 8, up4 = lane & 4, up2 = lane & 2;
#pragma unroll
    for (int m = 0; m < 4; ++m)
        v[m] = (up8 ? v[4 + m] : v[m]) + dpp_f<0x128>(up8 ? v[m] : v[4 + m]);
#pragma unroll
    for (int m = 0; m < 2; ++m)
        v[m] = (up4 ? v[2 + m] : v[m]) + u2f(__builtin_amdgcn_ds_swizzle((int)f2u(up4 ? v[m] : v[2 + m]), 0x101f));
    v[0] = (up2 ? v[1] : v[0]) + dpp_f<0x4e>(up2 ? v[0] : v[1]);
    return v[0] + dpp_f<0xb1>(v[0]);
}

template <bool XF>
__global__ __launch_bounds__(256) void prep_kernel_pk(PrepArgs a) {
    // ka: the A form of k for L, then that of q for P, then T (fp32 64 x 65);
    // kb: the B form of k, then the partial products of the inverse; Ls: the
    // gate's column sums until L is written; ft: the per-key factors f(I, J)
    __shared__ __attribute__((aligned(16))) f16 ka[BT * PKL];
    __shared__ __attribute__((aligned(16))) f16 kb[BT * PKL];
    __shared__ __attribute__((aligned(16))) float Ls[BT * LDL];
    __shared__ __attribute__((aligned(16))) f16 ft[10 * DK];
    __shared__ float bet[BT];
    float (*part)[DK] = reinterpret_cast<float (*)[DK]>(Ls);            // [4][DK] column sums of g per wave
    f16* qa = ka;
    float* Ts = reinterpret_cast<float*>(ka);
    float* Yb = reinterpret_cast<float*>(kb);

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = blockIdx.x, head = blockIdx.y, H = a.H;
    int u, cc;
    chunk_of(a.um, ci, u, cc);
    u = __builtin_amdgcn_readfirstlane(u);
    cc = __builtin_amdgcn_readfirstlane(cc);
    if (u < 0) return;
    const UnitInfo ui = uniform(unit_info(a.um, u));
    const int64_t t0 = ui.start + (int64_t)cc * BT;
    int len = ui.len - cc * BT;
    len = len < 0 ? 0 : (len > BT ? BT : len);
    const int64_t ch = (int64_t)ci * H + head;
    const int64_t e0 = t0 * H + head;              // token-head index of the chunk's first row
    const bool has_q = a.q != nullptr;
    const float l2b = a.use_exp2 ? 1.0f : 1.4426950408889634f;   // log2 of the decay base

    // ---- loads: buffer ranges end at the chunk's last token, so rows past it
    // read as zero (and the cumulative gate stays flat there)
    const uint32_t rowk = (uint32_t)H * DK * 2, rowg = (uint32_t)H * DK * 4;
    const rsrc_t rk = make_rsrc(reinterpret_cast<const bf16*>(a.k) + e0 * DK, len > 0 ? (uint32_t)(len - 1) * rowk + DK * 2 : 0);
    const rsrc_t rq = make_rsrc(has_q ? reinterpret_cast<const bf16*>(a.q) + e0 * DK : a.k,
                                has_q && len > 0 ? (uint32_t)(len - 1) * rowk + DK * 2 : 0);
    const rsrc_t rg = make_rsrc(a.g + e0 * DK, len > 0 ? (uint32_t)(len - 1) * rowg + DK * 4 : 0);
    uint32_t kr[16], qr[16];
    u32x2 gr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint32_t row = 16 * w + r;
        gr[r] = __builtin_amdgcn_raw_buffer_load_b64(rg, row * rowg + 8 * lane, 0, 0);
        kr[r] = __builtin_amdgcn_raw_buffer_load_b32(rk, row * rowk + 4 * lane, 0, 0);
        qr[r] = __builtin_amdgcn_raw_buffer_load_b32(rq, row * rowk + 4 * lane, 0, 0);
    }
    if (tid < BT) {
        float bt = tid < len ? (float)reinterpret_cast<const bf16*>(a.beta)[(t0 + tid) * H + head] : 0.0f;
        if (XF && a.beta_sig && tid < len) bt = sigmoid_f(bt);
        if (XF && a.beta_eff && tid < len) reinterpret_cast<bf16*>(a.beta_eff)[(t0 + tid) * H + head] = (bf16)bt;
        bet[tid] = bt;
        f16* cf = reinterpret_cast<f16*>(a.ws.cfh) + ch * (CFB / 2);
        const int lo = lane_order(tid);
        cf[CF_CY + lo] = (f16)bt;
        cf[CF_CP + lo] = (f16)1.0f;
        cf[CF_BG + lo] = (f16)1.0f;
        cf[CF_BETA + lo] = (f16)bt;
    }

    // ---- q / k normalisation: the reciprocal norm r of each of the wave's
    // rows (uniform), from one 64-lane reduction of all 32 sums of squares;
    // optional slots of the transformed rows
    float nk[16], nq[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) { nk[r] = 1.0f; nq[r] = 1.0f; }
    if (XF && a.qk_norm) {
        float v[32];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float k0 = __builtin_bit_cast(float, kr[r] << 16), k1 = __builtin_bit_cast(float, kr[r] & 0xffff0000u);
            const float q0 = __builtin_bit_cast(float, qr[r] << 16), q1 = __builtin_bit_cast(float, qr[r] & 0xffff0000u);
            v[r] = k0 * k0 + k1 * k1;
            v[16 + r] = q0 * q0 + q1 * q1;
        }
        const float s = lane_sum32(v, lane);   // sum m in lanes 2m, 2m + 1
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (16 * w + r < len) {
                nk[r] = rnorm_f(u2f(__builtin_amdgcn_readlane(f2u(s), 2 * r)));
                nq[r] = rnorm_f(u2f(__builtin_amdgcn_readlane(f2u(s), 32 + 2 * r)));
            }
    }
    if (XF && (a.k_hat || a.q_hat || a.k_rstd || a.q_rstd)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 16 * w + r;
            if (row >= len) continue;
            const int64_t re = e0 + (int64_t)row * H;
            auto rb = [](uint32_t x, float f) {
                const float lo = __builtin_bit_cast(float, x << 16) * f, hi = __builtin_bit_cast(float, x & 0xffff0000u) * f;
                return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)hi) << 16);
            };
            if (a.k_hat) reinterpret_cast<uint32_t*>(reinterpret_cast<bf16*>(a.k_hat) + re * DK)[lane] = rb(kr[r], nk[r]);
            if (has_q && a.q_hat) reinterpret_cast<uint32_t*>(reinterpret_cast<bf16*>(a.q_hat) + re * DK)[lane] = rb(qr[r], nq[r]);
            if (lane == 0 && a.k_rstd) a.k_rstd[re] = nk[r];
            if (lane == 0 && has_q && a.q_rstd) a.q_rstd[re] = nq[r];
        }
    }

    // ---- cumulative gate down each key column
    float gc[16][2];
    {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s0 += u2f(gr[r][0]);
            s1 += u2f(gr[r][1]);
            gc[r][0] = s0;
            gc[r][1] = s1;
        }
        part[w][2 * lane] = s0;
        part[w][2 * lane + 1] = s1;
    }
    lds_barrier();
    // rho_{w-1} (the sum of the blocks before), rho_w and G_L of this lane's keys
    float p0 = 0.0f, p1 = 0.0f, t0s = 0.0f, t1s = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
        const float x0 = part[ww][2 * lane], x1 = part[ww][2 * lane + 1];
        if (ww < w) { p0 += x0; p1 += x1; }
        t0s += x0;
        t1s += x1;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        gc[r][0] += p0;
        gc[r][1] += p1;
        const int row = 16 * w + r;
        if (a.g_cumsum && row < len)
            *reinterpret_cast<float2*>(a.g_cumsum + (e0 + (int64_t)row * H) * DK + 2 * lane) = float2{gc[r][0], gc[r][1]};
    }
    const float r0 = gc[15][0], r1 = gc[15][1];     // rho_w
    if (tid < DK) {
        float gl = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) gl += part[ww][tid];
        a.ws.gamL[ch * DK + tid] = gl;
        reinterpret_cast<float*>(a.ws.cfh)[ch * (CFB / 4) + CF_GL + tid] = fpow(gl, a.use_exp2);
    }
    // per-key factors f(I, J) = b^{rho_{I-1} - rho_J} of the 10 tiles J <= I
    for (int e = tid; e < 10 * DK; e += 256) {
        const int tri = e / DK, d = e % DK;
        const int I = tri < 1 ? 0 : tri < 3 ? 1 : tri < 6 ? 2 : 3, J = tri - I * (I + 1) / 2;
        float rI = 0.0f, rJ = 0.0f;
        for (int ww = 0; ww < 4; ++ww) {
            const float x = part[ww][d];
            if (ww < I) rI += x;
            if (ww <= J) rJ += x;
        }
        // diagonal factors beyond the factored range are never used
        ft[e] = (f16)fpow(fminf(rI - rJ, PK_DIAG_LOG2 / l2b), a.use_exp2);
    }

    // the diagonal tile's factored form needs the block's gate range within PK_DIAG_LOG2
    float rng = fmaxf(p0 - r0, p1 - r1) * l2b;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) rng = fmaxf(rng, __shfl_xor(rng, s, 64));
    const bool diag_direct = __builtin_amdgcn_readfirstlane(rng > PK_DIAG_LOG2 ? 1 : 0);
    // Direct diagonal tile: lanes 2m, 2m+1 end with value m of every row i
    // of the block, L_ij (m = j < 16; before beta) or P_ij (m = 16 + j)
    float dres[16];
    if (diag_direct) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float v[32];
#pragma unroll
            for (int m = 0; m < 32; ++m) v[m] = 0.0f;
            const float ki0 = __builtin_bit_cast(float, kr[i] << 16) * nk[i], ki1 = __builtin_bit_cast(float, kr[i] & 0xffff0000u) * nk[i];
            const float qi0 = __builtin_bit_cast(float, qr[i] << 16) * nq[i], qi1 = __builtin_bit_cast(float, qr[i] & 0xffff0000u) * nq[i];
#pragma unroll
            for (int j = 0; j <= i; ++j) {
                const float kj0 = __builtin_bit_cast(float, kr[j] << 16) * nk[j] * fpow(gc[i][0] - gc[j][0], a.use_exp2);
                const float kj1 = __builtin_bit_cast(float, kr[j] & 0xffff0000u) * nk[j] * fpow(gc[i][1] - gc[j][1], a.use_exp2);
                if (j < i) v[j] = ki0 * kj0 + ki1 * kj1;
                v[16 + j] = qi0 * kj0 + qi1 * kj1;
            }
            dres[i] = lane_sum32(v, lane);
        }
    }
    // ---- A and B forms to LDS (q's A form waits in registers until L is
    // done), the state pass's operands out
    uint32_t qpk[16];
    {
        const float cA0 = fpow(p0, a.use_exp2), cA1 = fpow(p1, a.use_exp2);                // b^{rho_{w-1}}
        const float cB0 = fpow(t0s - r0, a.use_exp2), cB1 = fpow(t1s - r1, a.use_exp2);    // b^{G_L - rho_w}
        const int cp = op_pos(2 * lane);
        uint32_t* qg = reinterpret_cast<uint32_t*>(reinterpret_cast<f16*>(a.ws.qg) + ch * (BT * DK) + cp);
        uint32_t* kd = reinterpret_cast<uint32_t*>(reinterpret_cast<f16*>(a.ws.kd) + ch * (BT * DK) + cp);
        uint32_t* kg = reinterpret_cast<uint32_t*>(reinterpret_cast<f16*>(a.ws.kg) + ch * (BT * DK) + cp);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 16 * w + r;
            const float k0 = __builtin_bit_cast(float, kr[r] << 16) * nk[r], k1 = __builtin_bit_cast(float, kr[r] & 0xffff0000u) * nk[r];
            const float q0 = __builtin_bit_cast(float, qr[r] << 16) * nq[r], q1 = __builtin_bit_cast(float, qr[r] & 0xffff0000u) * nq[r];
            const float eA0 = fpow(gc[r][0] - p0, a.use_exp2), eA1 = fpow(gc[r][1] - p1, a.use_exp2);
            const float eB0 = fpow(r0 - gc[r][0], a.use_exp2), eB1 = fpow(r1 - gc[r][1], a.use_exp2);
            const float ka0 = k0 * eA0, ka1 = k1 * eA1, qa0 = q0 * eA0, qa1 = q1 * eA1;
            const float kb0 = k0 * eB0, kb1 = k1 * eB1;
            *reinterpret_cast<uint32_t*>(&ka[row * PKL + 2 * lane]) = pack_f16x2(ka0, ka1);
            *reinterpret_cast<uint32_t*>(&kb[row * PKL + 2 * lane]) = pack_f16x2(kb0, kb1);
            qpk[r] = pack_f16x2(qa0, qa1);
            if (has_q) qg[row * (DK / 2)] = pack_f16x2(qa0 * cA0, qa1 * cA1);
            kd[row * (DK / 2)] = pack_f16x2(ka0 * cA0, ka1 * cA1);
            kg[row * (DK / 2)] = pack_f16x2(kb0 * cB0, kb1 * cB1);
        }
    }
    lds_barrier();

    // ---- L (strictly lower) and P (lower incl. diagonal) on MFMA, with the
    // tile coordinates of each wave fixed at compile time: tile (I, J) pairs
    // the A forms of rows I with the B form of rows J scaled by f(I, J) (no
    // scaling for J = I - 1, where f = 1)
    f16* Pw = reinterpret_cast<f16*>(a.ws.P) + ch * (BT * BT);
    auto tiles = [&](auto w_c) {
        constexpr int WV = decltype(w_c)::value;
        auto bfrag = [&](auto I_c, auto J_c, int kk) {
            constexpr int I = decltype(I_c)::value, J = decltype(J_c)::value;
            const int col = 32 * kk + 8 * G;
            PolicyH::F r;
            r.v = *reinterpret_cast<const f16x8*>(&kb[(16 * J + n) * PKL + col]);
            if (J != I - 1) r.v = r.v * *reinterpret_cast<const f16x8*>(&ft[pk_tri(I, J) * DK + col]);
            return r;
        };
        // L
        auto ltile = [&](auto s_c) {
            constexpr int S = decltype(s_c)::value;
            constexpr int I = PK_TI[WV][S], J = PK_TJ[WV][S];
            if (I == J && diag_direct) {
                const int m = lane >> 1, j = m & 15;
                if (!(lane & 1) && m < 16)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        Ls[(16 * I + i) * LDL + 16 * I + j] = j < i ? bet[16 * I + i] * dres[i] : 0.0f;
                return;
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                PolicyH::mma(acc, PolicyH::ld(&ka[(16 * I + n) * PKL + 32 * kk + 8 * G]),
                             bfrag(std::integral_constant<int, I>{}, std::integral_constant<int, J>{}, kk));
            // acc[r]: row i = 16 I + 4G + r against column j = 16 J + n
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int il = 4 * G + r, i = 16 * I + il;
                float x = bet[i] * acc[r];
                if (I == J) x = n < il ? x : 0.0f;
                Ls[i * LDL + 16 * J + n] = x;
            }
        };
        ltile(std::integral_constant<int, 0>{});
        ltile(std::integral_constant<int, 1>{});
        if constexpr (PK_NT[WV] > 2) ltile(std::integral_constant<int, 2>{});
        lds_barrier();
        // q's A form over k's, which L no longer needs
        if (has_q) {
#pragma unroll
            for (int r = 0; r < 16; ++r) *reinterpret_cast<uint32_t*>(&qa[(16 * WV + r) * PKL + 2 * lane]) = qpk[r];
        }
        lds_barrier();
        if (!has_q) return;
        // P, and the zero tiles above the diagonal
#pragma unroll
        for (int z = PK_Z0[WV]; z < PK_Z0[WV] + PK_NZ[WV]; ++z) {             // (it, jt) with it < jt
            const int it = z < 3 ? 0 : (z < 5 ? 1 : 2);
            const int jt = z < 3 ? z + 1 : (z < 5 ? z - 1 : 3);
            *reinterpret_cast<u32x2*>(Pw + (16 * it + n) * BT + op_pos(16 * jt + 4 * G)) = u32x2{0u, 0u};
        }
        auto ptile = [&](auto s_c) {
            constexpr int S = decltype(s_c)::value;
            constexpr int I = PK_TI[WV][S], J = PK_TJ[WV][S];
            if (I == J && diag_direct) {
                const int m = lane >> 1, j = m & 15;
                if (!(lane & 1) && m >= 16)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        Pw[(16 * I + i) * BT + op_pos(16 * I + j)] = (f16)(j <= i ? dres[i] : 0.0f);
                return;
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                PolicyH::mma(acc, bfrag(std::integral_constant<int, I>{}, std::integral_constant<int, J>{}, kk),
                             PolicyH::ld(&qa[(16 * I + n) * PKL + 32 * kk + 8 * G]));
            // acc[r]: row i = 16 I + n against column j = 16 J + 4G + r
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (I > J || 4 * G + r <= n) ? acc[r] : 0.0f;
            PolicyH::st4(Pw + (16 * I + n) * BT + op_pos(16 * J + 4 * G), x);
        };
        ptile(std::integral_constant<int, 0>{});
        ptile(std::integral_constant<int, 1>{});
        if constexpr (PK_NT[WV] > 2) ptile(std::integral_constant<int, 2>{});
    };
    if (w == 0) tiles(std::integral_constant<int, 0>{});
    else if (w == 1) tiles(std::integral_constant<int, 1>{});
    else if (w == 2) tiles(std::integral_constant<int, 2>{});
    else tiles(std::integral_constant<int, 3>{});
    lds_barrier();

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
        for (int e = tid - 64; e < 6 * 256; e += 192) {
            const int blk = e >> 8, rr = (e >> 4) & 15, cc2 = e & 15;
            const int I = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
            const int J = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
            Ts[(16 * I + rr) * LDL + 16 * J + cc2] = 0.0f;
        }
    }
    lds_barrier();
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
        lds_barrier();
        for (int e = tid; e < nb * 256; e += 256) {
            const int bi = e >> 8, rr = (e >> 4) & 15, cc2 = e & 15;
            const int I = d + bi, J = bi;
            float s = 0.0f;
            for (int m = 0; m < 16; ++m) s += Ts[(16 * I + rr) * LDL + 16 * I + m] * Yb[(bi * 16 + m) * 17 + cc2];
            Ts[(16 * I + rr) * LDL + 16 * J + cc2] = -s;
        }
        lds_barrier();
    }

    // ---- T out as fp16 operands (op_pos columns), optional token-major fp32 A slot
    f16* Tw = reinterpret_cast<f16*>(a.ws.Tm) + ch * (BT * BT);
    for (int e = tid; e < BT * BT / 4; e += 256) {
        const int r = e / (BT / 4), c4 = (e % (BT / 4)) * 4;
        f32x4 x;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) x[q2] = Ts[r * LDL + c4 + q2];
        PolicyH::f32_to_op4(Tw + r * BT + op_pos(c4), x);
        if (a.A && r < len) *reinterpret_cast<f32x4*>(a.A + (e0 + (int64_t)r * H) * BT + c4) = x;
    }
}

// ------------------------------------------------------------------ state pass
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
    int tile0;       // first column tile (summary mode: 0, or the first M tile)
    float* S_ext;
    float* M;
    const int32_t* order;   // units in launch order (longest first), or NULL: natural order
    float* vnew;            // optional slot: v_new, fp32 [tokens][H][V]
    int beta_sig;           // beta through a sigmoid (the fp32 pass, which reads beta itself)
};

// Work split of the 8 waves of a state-pass workgroup (one 32-column value
// tile): wave w owns token rows 16*rg .. 16*rg+15 and state rows (keys)
// 32*rg .. 32*rg+31 of row group rg, and the 16 value columns of column group
// cg. Waves w and w+4 share a SIMD; pairing row group s with 3-s there
// balances the triangular work (later rows of a chunk see more of it).
constexpr int SW = 8;              // waves per state-pass workgroup
constexpr int ST = 64 * SW;        // threads
constexpr int LDY = BT + 8;        // rows (value columns) of the transposed 64-token LDS tiles

template <class P, bool PERKEY, bool SUMMARY>
__global__ __launch_bounds__(ST) void state_kernel(StateArgs a) {
    using In = typename P::In;
    using Op = typename P::Op;
    using F = typename P::F;
    constexpr int LDQ = P::LDQ;
    constexpr int FV = P::FV;
    constexpr bool OUT = !SUMMARY;
    // Each wave reads its q, T and P rows into registers and stores its
    // output rows directly; k and the per-key gated k are shared through LDS.
    __shared__ __attribute__((aligned(16))) Op kt[2][BT * LDQ];                  // k (per key: k*b^G)
    __shared__ __attribute__((aligned(16))) Op kgt[PERKEY ? BT * LDQ : 8];       // per key: k*b^{G_last-G}
    __shared__ __attribute__((aligned(16))) Op hT[BV * LDQ];                     // state, transposed
    __shared__ __attribute__((aligned(16))) Op YT[BV * LDY];
    __shared__ __attribute__((aligned(16))) Op vnT[OUT ? BV * LDY : 8];
    __shared__ __attribute__((aligned(16))) Op vpT[BV * LDY];
    __shared__ __attribute__((aligned(16))) float gam[2][GAMR * BT];             // G, b^G r_k, b^{G_L-G} r_k, b^{G_L}, b^G r_q
    __shared__ __attribute__((aligned(16))) float bet[2][BT];
    __shared__ __attribute__((aligned(16))) float gl[2][PERKEY ? DK : 4];

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);          // wave index, kept scalar
    const int cg = wv >> 2;                                           // column group
    const int rg = cg == 0 ? (wv & 3) : 3 - (wv & 3);                 // row group
    const int H = a.H;
    // blocks are dealt round-robin to the 8 XCDs: keep every column tile of a
    // (unit, head) pair on one XCD so that they share its L2
    const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
    const int tile = slot % a.ntiles + a.tile0;
    const int pair = (slot / a.ntiles) * 8 + xcd;
    if (pair >= a.n_pairs) return;
    const int pu = pair / H, head = pair - pu * H;
    const int u = a.order ? a.order[pu] : pu;
    if ((unsigned)u >= (unsigned)a.um.n_units) return;
    const UnitInfo ui = unit_info(a.um, u);
    const int c0 = tile * BV;                       // column of [S_ext | M] or of V
    const bool mcols = SUMMARY && c0 >= DV;         // transfer-map columns: v = 0, start at I
    const int vc0 = mcols ? c0 - DV : c0;           // first state / output column of the workgroup
    const int col = vc0 + 16 * cg + n;              // this lane's state / output column
    const In* qin = reinterpret_cast<const In*>(a.q);
    const In* kin = reinterpret_cast<const In*>(a.k);
    const In* vin = reinterpret_cast<const In*>(a.v);
    const In* bin = reinterpret_cast<const In*>(a.beta);
    const int nkw = rg >= 2 ? 2 : 1;                // 32-token steps that cover rows <= 16rg+15
    const int e2 = a.use_exp2;
    const uint32_t tokstride = (uint32_t)H * DK;    // elements between consecutive tokens (K = V)

    // ---- state tile: rows (keys) 32rg + 16ks + 4G + r, column col
    f32x4 h[2];
    for (int ks = 0; ks < 2; ++ks)
        for (int r = 0; r < 4; ++r) {
            const int key = 32 * rg + 16 * ks + 4 * G + r;
            float x = 0.0f;
            if (mcols) x = key == col ? 1.0f : 0.0f;
            else if (OUT && a.h0) x = a.h0[(((int64_t)u * H + head) * DK + key) * DV + col];
            h[ks][r] = x;
        }

    // ---- next-chunk prefetch. Loads for chunk c+1 are issued at the start of
    // step c and stay raw in registers until published (k, q, T and the gates
    // at the end of step c, P and the per-key gated k at the start of step
    // c+1), so their latency overlaps a whole step. Every tile load is a
    // contiguous 16 bytes per lane. Rows past the chunk end read a clamped
    // (valid) row: their contributions vanish because beta is zero there and
    // T is the identity on padded rows, and padded output rows are not stored.
    constexpr int VPR = 16 / sizeof(In);
    constexpr int NKV = BT * DK / VPR / ST;           // 16-byte vectors per thread of a 64 x 128 tile
    constexpr int NGW = PERKEY ? DK : GAMR * BT;      // gate words per chunk
    constexpr int RQ = 4 * FV;                        // q registers: the wave's rows
    constexpr int RT = 2 * FV;                        // T / P registers: the wave's rows
    auto chunk_len = [&](int c) { int l = ui.len - c * BT; return l < 0 ? 0 : (l > BT ? BT : l); };
    struct Raw {
        f32x4 k[NKV];                    // k tile (per key: k*b^G operands)
        f32x4 q[OUT ? RQ : 1];           // q (per key: q*b^G operands)
        f32x4 T[RT];                     // T operands
        f32x4 Pr[OUT ? RT : 1];          // P operands
        f32x4 kg[PERKEY ? NKV : 1];      // per key: k*b^{G_last-G} operands
        float gb;                        // gate word tid (threads < NGW)
        In bt;                           // beta
        In v[4];                         // v rows 16rg+4G+r, column col
        int len;
    };
    auto tile_rc = [&](int i, int& r, int& cv) {     // 64 x 128 tile vector -> (row, column)
        const int idx = tid + ST * i;
        r = idx / (DK / VPR);
        cv = (idx % (DK / VPR)) * VPR;
    };
    auto load_raw = [&](int c, Raw& x) {
        const int len = chunk_len(c);
        x.len = len;
        const int last = len > 0 ? len - 1 : 0;
        const int64_t t0 = ui.start + (int64_t)c * BT;
        const int64_t ch = (int64_t)(ui.cbase + c) * H + head;
        const int row = 16 * rg + n;
        const Op* Tw = reinterpret_cast<const Op*>(a.ws.Tm) + ch * (BT * BT);
        const Op* Pw = reinterpret_cast<const Op*>(a.ws.P) + ch * (BT * BT);
        if (PERKEY) {
            const Op* kd = reinterpret_cast<const Op*>(a.ws.kd) + ch * (BT * DK);
            const Op* kg = reinterpret_cast<const Op*>(a.ws.kg) + ch * (BT * DK);
            for (int i = 0; i < NKV; ++i) {
                int r, cv;
                tile_rc(i, r, cv);
                x.k[i] = *reinterpret_cast<const f32x4*>(kd + r * DK + cv);
                x.kg[i] = *reinterpret_cast<const f32x4*>(kg + r * DK + cv);
            }
            x.gb = tid < NGW ? a.ws.gamL[ch * DK + tid] : 0.0f;
        } else {
            const In* kb = kin + (t0 * H + head) * DK;
            for (int i = 0; i < NKV; ++i) {
                int r, cv;
                tile_rc(i, r, cv);
                x.k[i] = *reinterpret_cast<const f32x4*>(kb + (uint32_t)min(r, last) * tokstride + cv);
            }
            x.gb = tid < NGW ? a.ws.gam[ch * (GAMR * BT) + tid] : 0.0f;
        }
        if (OUT) {
            const Op* qg = reinterpret_cast<const Op*>(a.ws.qg) + ch * (BT * DK);
            const In* qb = qin + (t0 * H + head) * DK;
            for (int kk = 0; kk < 4; ++kk)
                for (int f = 0; f < FV; ++f)
                    x.q[FV * kk + f] = PERKEY ? *reinterpret_cast<const f32x4*>(qg + row * DK + 32 * kk + 8 * G + 4 * f)
                                              : *reinterpret_cast<const f32x4*>(qb + (uint32_t)min(row, last) * tokstride +
                                                                                 32 * kk + 8 * G + 4 * f);
        }
        for (int kk = 0; kk < 2; ++kk)
            if (kk < nkw)
                for (int f = 0; f < FV; ++f) {
                    x.T[FV * kk + f] = *reinterpret_cast<const f32x4*>(Tw + row * BT + 32 * kk + 8 * G + 4 * f);
                    if (OUT) x.Pr[FV * kk + f] = *reinterpret_cast<const f32x4*>(Pw + row * BT + 32 * kk + 8 * G + 4 * f);
                }
        x.bt = (bin + t0 * H + head)[(uint32_t)min(lane, last) * H];
        if (!mcols) {
            const In* vb = vin + (t0 * H + head) * DV;
            for (int r = 0; r < 4; ++r) x.v[r] = vb[(uint32_t)min(16 * rg + 4 * G + r, last) * tokstride + col];
        }
    };
    // k, q, T and the gates of a chunk (read from its step's start)
    auto publish_main = [&](const Raw& x, int b) {
        for (int i = 0; i < NKV; ++i) {
            int r, cv;
            tile_rc(i, r, cv);
            *reinterpret_cast<f32x4*>(&kt[b][r * LDQ + cv]) = PERKEY ? x.k[i] : P::in2op(x.k[i]);
        }
        if (tid < NGW) {
            if (PERKEY) gl[b][tid] = x.gb;
            else gam[b][tid] = x.gb;
        }
        if (tid < BT) bet[b][tid] = tid < x.len ? (a.beta_sig ? sigmoid_f(P::f(x.bt)) : P::f(x.bt)) : 0.0f;
    };
    // the per-key gated k of a chunk (read only after its step's first barrier)
    auto publish_late = [&](const Raw& x) {
        if (PERKEY)
            for (int i = 0; i < NKV; ++i) {
                int r, cv;
                tile_rc(i, r, cv);
                *reinterpret_cast<f32x4*>(&kgt[r * LDQ + cv]) = x.kg[i];
            }
    };
    // ---- prologue
    const int nch = ui.nch;
    Raw cur, nxt;
    if (nch > 0) {
        load_raw(0, cur);
        publish_main(cur, 0);
    }
    for (int ks = 0; ks < 2; ++ks) {
        float x[4] = {h[ks][0], h[ks][1], h[ks][2], h[ks][3]};
        P::st4(&hT[(16 * cg + n) * LDQ + 32 * rg + 16 * ks + 4 * G], x);
    }
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        const int len = cur.len;
        const int64_t t0 = ui.start + (int64_t)c * BT;
        const int64_t ch = (int64_t)(ui.cbase + c) * H + head;
        const bool more = c + 1 < nch;
        publish_late(cur);
        if (more) load_raw(c + 1, nxt);
        if (OUT && a.hslot) {
            for (int ks = 0; ks < 2; ++ks)
                for (int r = 0; r < 4; ++r) {
                    const int key = 32 * rg + 16 * ks + 4 * G + r;
                    a.hslot[((ch * DK) + key) * DV + col] = h[ks][r];
                }
        }
        const float* gm = gam[b];
        const f32x4 eG = PERKEY ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&gm[BT + 16 * rg + 4 * G]);
        const f32x4 eLG = PERKEY ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&gm[2 * BT + 16 * rg + 4 * G]);

        // ---- token side: K h and q h for rows 16rg .. 16rg+15, columns of cg
        const Op* K = kt[b];
        f32x4 kh = {0.f, 0.f, 0.f, 0.f}, qh = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < 4; ++kk) {
            const F hb = P::ld(&hT[(16 * cg + n) * LDQ + 32 * kk + 8 * G]);
            P::mma(kh, P::ld(&K[(16 * rg + n) * LDQ + 32 * kk + 8 * G]), hb);
            if (OUT) {
                f32x4 qv[FV];
                for (int f = 0; f < FV; ++f) qv[f] = PERKEY ? cur.q[FV * kk + f] : P::in2op(cur.q[FV * kk + f]);
                P::mma(qh, P::frag(qv), hb);
            }
        }
        // Y = beta (v - b^G K h) (per key: K already carries b^G)
        {
            const f32x4 bt = *reinterpret_cast<const f32x4*>(&bet[b][16 * rg + 4 * G]);
            float y[4];
            for (int r = 0; r < 4; ++r) {
                const float vv = mcols ? 0.0f : P::f(cur.v[r]);
                y[r] = bt[r] * (vv - eG[r] * kh[r]);
            }
            P::st4(&YT[(16 * cg + n) * LDY + 16 * rg + 4 * G], y);
        }
        f32x4 oacc;
        if (OUT) {
            const f32x4 eQ = PERKEY ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&gm[4 * BT + 16 * rg + 4 * G]);
            for (int r = 0; r < 4; ++r) oacc[r] = eQ[r] * qh[r];
        }
        __syncthreads();

        // ---- v_new = T Y for rows 16rg .. 16rg+15
        f32x4 vn = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < 2; ++kk)
            if (kk < nkw) {
                const F ta = P::frag(&cur.T[FV * kk]);
                P::mma(vn, ta, P::ld(&YT[(16 * cg + n) * LDY + 32 * kk + 8 * G]));
            }
        if (OUT && a.vnew)
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * rg + 4 * G + r;
                if (i < len) a.vnew[((t0 + i) * H + head) * DV + col] = vn[r];
            }
        {
            float x[4], xp[4];
            for (int r = 0; r < 4; ++r) {
                x[r] = vn[r];
                xp[r] = vn[r] * eLG[r];
            }
            if (OUT) P::st4(&vnT[(16 * cg + n) * LDY + 16 * rg + 4 * G], x);
            P::st4(&vpT[(16 * cg + n) * LDY + 16 * rg + 4 * G], xp);
        }
        __syncthreads();

        // ---- output rows 16rg .. 16rg+15
        if (OUT) {
            for (int kk = 0; kk < 2; ++kk)
                if (kk < nkw) {
                    P::mma(oacc, P::frag(&cur.Pr[FV * kk]), P::ld(&vnT[(16 * cg + n) * LDY + 32 * kk + 8 * G]));
                }
            float* of = reinterpret_cast<float*>(a.o) + (t0 * H + head) * DV;
            bf16* ob = reinterpret_cast<bf16*>(a.o) + (t0 * H + head) * DV;
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * rg + 4 * G + r;
                if (i < len) {
                    const float x = a.scale * oacc[r];
                    const uint32_t off = (uint32_t)i * tokstride + col;
                    if (a.o_bf16) ob[off] = (bf16)x;
                    else of[off] = x;
                }
            }
        }

        // ---- state: h = Diag(b^{G_last}) h + kg^T v_new' for keys 32rg .. 32rg+31
        {
            F vb[2];
            for (int kk = 0; kk < 2; ++kk) vb[kk] = P::ld(&vpT[(16 * cg + n) * LDY + 32 * kk + 8 * G]);
            const Op* KG = PERKEY ? kgt : K;
            for (int ks = 0; ks < 2; ++ks) {
                if (PERKEY) {
                    const f32x4 gv = *reinterpret_cast<const f32x4*>(&gl[b][32 * rg + 16 * ks + 4 * G]);
                    for (int r = 0; r < 4; ++r) h[ks][r] *= fpow(gv[r], e2);
                } else {
                    const float eL = gm[3 * BT];
                    for (int r = 0; r < 4; ++r) h[ks][r] *= eL;
                }
                for (int kk = 0; kk < 2; ++kk) P::mma(h[ks], P::ldcol(KG, LDQ, 32 * kk, 32 * rg + 16 * ks, lane), vb[kk]);
                float x[4] = {h[ks][0], h[ks][1], h[ks][2], h[ks][3]};
                P::st4(&hT[(16 * cg + n) * LDQ + 32 * rg + 16 * ks + 4 * G], x);
            }
        }
        if (more) {
            publish_main(nxt, b ^ 1);
            cur = nxt;
        }
        __syncthreads();
    }

    // ---- results
    for (int ks = 0; ks < 2; ++ks)
        for (int r = 0; r < 4; ++r) {
            const int key = 32 * rg + 16 * ks + 4 * G + r;
            const int64_t uh = (int64_t)u * H + head;
            if (SUMMARY) {
                if (mcols) { if (a.M) a.M[(uh * DK + key) * DK + col] = h[ks][r]; }
                else if (a.S_ext) a.S_ext[(uh * DK + key) * DV + col] = h[ks][r];
            } else if (a.hfinal) {
                a.hfinal[(uh * DK + key) * DV + col] = h[ks][r];
            }
        }
}

// ------------------------------------------------------------------ state pass, split keys (bf16)
// Workgroup of 8 waves for one (unit, head, 32-column tile). Compute wave
// w < 4 owns value columns 16 (w & 1) .. +15 and keys 64 (w >> 1) .. +63 of
// the fp32 state, so the four compute waves run on all four SIMDs. At the
// end of each step a wave publishes its keys' half of the fp16 state operand
// in LDS; after the barrier its partner (w ^ 2) reads it, so both hold the
// whole operand and form k.h for all 64 rows themselves (the products are
// duplicated, the step needs no second barrier). Each wave then builds Y and
// v_new = T Y for all rows, updates its own keys, and computes the output rows
// of its half (rows 0..31 for the first key half, 32..63 for the second).
// Waves 4..7 stream the tiles with ordinary buffer loads into registers and
// write them to double-buffered LDS, each a quarter of the token rows of
// every tile: k and q (converted to fp16 operands in op_pos order), T, P and
// the v rows of the column tile, plus the coefficient block. Each holds two
// register sets, so the loads of chunk c+2 are issued at the start of step
// c, a full step before they are written out. Rows past the chunk end read
// as zero. The compute waves leave their output rows in an LDS tile; one
// step later the streaming waves store them as whole 128-byte row segments.
// Per-key gate (PK): the streaming waves copy the prepared k b^G, q b^G and
// k b^{G_L - G} tiles (already fp16 in op_pos order) into the same layout;
// k.h uses k b^G, the update uses k b^{G_L - G} and decays each key by its
// own b^{G_L}, the output uses q b^G. The third tile leaves no room for the
// output staging, so the compute waves store their output rows themselves.
constexpr int KSW = 8;
constexpr int OXP = BV + 4;        // row pitch (floats) of the output tile
constexpr int KST = 64 * KSW;

template <bool SUMMARY, bool OBF, bool PK>
__global__ __launch_bounds__(KST) void state_kernel_ks(StateArgs a) {
    using F = PolicyH::F;
    constexpr bool OUT = !SUMMARY;
    constexpr bool OXS = OUT && !PK;    // output rows staged in LDS (scalar gate)
    __shared__ __attribute__((aligned(16))) f16 kt[2][BT * DK];                   // k, or per key k b^G
    __shared__ __attribute__((aligned(16))) f16 qt[OUT ? 2 : 1][OUT ? BT * DK : 8];   // q, or q b^G
    __shared__ __attribute__((aligned(16))) f16 gt[PK ? 2 : 1][PK ? BT * DK : 8];     // per key: k b^{G_L - G}
    __shared__ __attribute__((aligned(16))) f16 Tt[2][BT * BT];
    __shared__ __attribute__((aligned(16))) f16 Pt[OUT ? 2 : 1][OUT ? BT * BT : 8];
    __shared__ __attribute__((aligned(16))) bf16 vt[2][BT * BV];
    __shared__ __attribute__((aligned(16))) float cb[2][CFS / 4];
    __shared__ __attribute__((aligned(16))) f16x8 hx[2][4][2][64];   // [step parity][wave][slice][lane]
    __shared__ __attribute__((aligned(16))) float ox[OXS ? 2 : 1][OXS ? BT * OXP : 4];   // scaled output rows

    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, n = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H;
    const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
    const int tile = slot % a.ntiles + a.tile0;
    const int pair = (slot / a.ntiles) * 8 + xcd;
    if (pair >= a.n_pairs) return;
    const int pu = pair / H, head = pair - pu * H;
    const int u = a.order ? a.order[pu] : pu;
    if ((unsigned)u >= (unsigned)a.um.n_units) return;
    const UnitInfo ui = uniform(unit_info(a.um, u));
    const int c0 = tile * BV;
    const bool mcols = SUMMARY && c0 >= DV;         // transfer-map columns: v = 0, start at I
    const int vc0 = mcols ? c0 - DV : c0;
    const int nch = ui.nch;
    const uint32_t tokstride = (uint32_t)H * DK;
    auto chunk_len = [&](int c) {
        int l = ui.len - c * BT;
        return __builtin_amdgcn_readfirstlane(l < 0 ? 0 : (l > BT ? BT : l));
    };

    // the compute body, instantiated per key half so that every register
    // array index is a compile-time constant
    auto compute = [&](auto kq_c) {
        constexpr int kq = decltype(kq_c)::value;
        const int cg = wv & 1, partner = wv ^ 2;
        const int col = vc0 + 16 * cg + n;
        const int64_t uh = (int64_t)u * H + head;
        f32x4 h[4];                                  // keys 64 kq + 16 j + 4G + r, column col
        for (int j = 0; j < 4; ++j)
            for (int r = 0; r < 4; ++r) {
                const int key = 64 * kq + 16 * j + 4 * G + r;
                float x = 0.0f;
                if (mcols) x = key == col ? 1.0f : 0.0f;
                else if (OUT && a.h0) x = a.h0[(uh * DK + key) * DV + col];
                h[j][r] = x;
            }
        auto pack = [](const f32x4& x, const f32x4& y) {
            F f;
            for (int e = 0; e < 4; ++e) { f.v[e] = (f16)x[e]; f.v[e + 4] = (f16)y[e]; }
            return f;
        };
        // the state operand, halves swapped on odd lane groups (the k and q tile layout)
        const bool hswap = G & 1;
        auto pack_state = [&](const f32x4& x, const f32x4& y) {
            const F f = pack(x, y);
            const u32x4 w = __builtin_bit_cast(u32x4, f.v);
            const u32x4 sw = {w[2], w[3], w[0], w[1]};
            F r;
            r.v = __builtin_bit_cast(f16x8, hswap ? sw : w);
            return r;
        };
        F hb[4];                                     // operand slices 0..3 (2 kq, 2 kq + 1 are this wave's)
        for (int j2 = 0; j2 < 2; ++j2) {
            hb[2 * kq + j2] = pack_state(h[2 * j2], h[2 * j2 + 1]);
            hx[0][wv][j2][lane] = hb[2 * kq + j2].v;
        }
        // per-lane LDS byte offsets
        int offA[4], offG[2];
        for (int s2 = 0; s2 < 4; ++s2) offA[s2] = n * 256 + (((4 * s2 + G) ^ swzk(n)) << 4);   // row n, granule 4 s2 + G
        for (int j2 = 0; j2 < 2; ++j2) {
            const int s2 = 2 * kq + j2, rt = 4 * G + (n >> 2);                  // transposed read row
            offG[j2] = rt * 256 + (((4 * s2 + (n & 3)) ^ swzk(rt)) << 4);
        }
        const int hlo = (n & 1) * 8;                 // byte offset of logical half 0 in granule 4 s2 + (n & 3)
        int offT[2];
        for (int kk = 0; kk < 2; ++kk) offT[kk] = n * 128 + (((4 * kk + G) ^ swz8(n)) << 4);
        const int offV = (4 * G + (n >> 2)) * (BV * 2) + 32 * cg + 8 * (n & 3);
        auto ldA = [](const f16* t, int byte_off) {
            F f;
            f.v = *reinterpret_cast<const f16x8*>(reinterpret_cast<const char*>(t) + byte_off);
            return f;
        };
        // k^T fragment of key tile 4 kq + j (keys 16 j + n of the wave's half)
        auto ldKT = [&](const f16* t, int j, int kk) {
            const char* p = reinterpret_cast<const char*>(t) + offG[j >> 1] + ((j & 1) * 8 ^ hlo) + kk * 32 * 256;
            s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p));
            s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p + 16 * 256));
            f16x4 fx = __builtin_bit_cast(f16x4, x), fy = __builtin_bit_cast(f16x4, y);
            F f;
            for (int e = 0; e < 4; ++e) { f.v[e] = fx[e]; f.v[e + 4] = fy[e]; }
            return f;
        };
        uint32_t hoff[4];
        for (int r = 0; r < 4; ++r) hoff[r] = (uint32_t)(64 * kq + 4 * G + r) * DV + col;
        lds_barrier();                              // chunk 0 and the entry state published

        for (int c = 0; c < nch; ++c) {
            const int cu = __builtin_amdgcn_readfirstlane(c);
            const int tb = cu & 1, tq = tb;
            const int len = chunk_len(cu);
            const int64_t t0 = ui.start + (int64_t)cu * BT;
            const int64_t ch = (int64_t)(ui.cbase + cu) * H + head;
            if (OUT && a.hslot) {
                float* hs = a.hslot + ch * (DK * DV);
                for (int j = 0; j < 4; ++j)
                    for (int r = 0; r < 4; ++r) hs[16 * j * DV + hoff[r]] = h[j][r];
            }
            const f16* K = kt[tb];
            const f16* KG = PK ? gt[tb] : kt[tb];    // keys of the state update
            const f16* Q = qt[OUT ? tq : 0];
            const f16* Tc = Tt[tb];
            const f16* Pc = Pt[OUT ? tb : 0];
            // the partner's half of the state operand
            for (int j2 = 0; j2 < 2; ++j2) hb[2 * (1 - kq) + j2].v = hx[tq][partner][j2][lane];
            // per-row coefficients: lane G holds rows 16 it + 4G + r at [16G + 4it + r]
            const float* cf = cb[tb];
            // scalar gate: b^{G_L - G}, b^G per row, b^{G_L}; per key: beta per
            // row (fp16) and b^{G_L} of this wave's keys
            f32x4 cpf[4], bg[4], gl[4];
            float eL = 1.0f;
            if (!PK) {
                for (int it = 0; it < 4; ++it) {
                    cpf[it] = *reinterpret_cast<const f32x4*>(&cf[CS_CP + 16 * G + 4 * it]);
                    bg[it] = *reinterpret_cast<const f32x4*>(&cf[CS_BG + 16 * G + 4 * it]);
                }
                eL = cf[CS_EL];
            } else {
                const f16* cbh = reinterpret_cast<const f16*>(cf);
                for (int it = 0; it < 4; ++it) {
                    const f16x4 b4 = *reinterpret_cast<const f16x4*>(&cbh[CF_BETA + 16 * G + 4 * it]);
                    for (int r = 0; r < 4; ++r) bg[it][r] = (float)b4[r];
                }
                for (int j = 0; j < 4; ++j) gl[j] = *reinterpret_cast<const f32x4*>(&cf[CF_GL + 64 * kq + 16 * j + 4 * G]);
            }
            s16x4 vraw[4];
            for (int it = 0; it < 4; ++it)
                vraw[it] = mcols ? s16x4{0, 0, 0, 0}
                                 : __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       LDS_PTR(s16x4, reinterpret_cast<const char*>(vt[tb]) + offV + it * 16 * BV * 2));

            // The step runs as a pipeline over the two 32-row halves: T is
            // lower triangular, so v_new of rows 0..31 needs Y of rows 0..31
            // only, and the state update from the first 32 tokens can run
            // while the k.h products of the second half complete.
            auto khY = [&](int it, f32x4& y) {           // Y = v - b^G (k h), row tile it (beta is in T)
                f32x4 kh = {0.f, 0.f, 0.f, 0.f};
                for (int s2 = 0; s2 < 4; ++s2) PolicyH::mma(kh, ldA(K, offA[s2] + it * 16 * 256), hb[s2]);
                for (int r = 0; r < 4; ++r) {
                    const float vv = __builtin_bit_cast(float, (uint32_t)(uint16_t)vraw[it][r] << 16);
                    y[r] = PK ? bg[it][r] * (vv - kh[r]) : __builtin_fmaf(-bg[it][r], kh[r], vv);
                }
            };
            f32x4 y[4], vn[4], vp[4];
            khY(0, y[0]);
            khY(1, y[1]);
            const F yb0 = pack(y[0], y[1]);
            for (int it = 0; it < 4; ++it) {
                vn[it] = f32x4{0.f, 0.f, 0.f, 0.f};
                PolicyH::mma(vn[it], ldA(Tc, offT[0] + it * 16 * 128), yb0);
            }
            khY(2, y[2]);
            khY(3, y[3]);
            // ---- state of this wave's keys: h = b^{G_L} h + kg^T v_new'
            for (int it = 0; it < 2; ++it)
                for (int r = 0; r < 4; ++r) vp[it][r] = PK ? vn[it][r] : vn[it][r] * cpf[it][r];
            const F vb0 = pack(vp[0], vp[1]);
            for (int j = 0; j < 4; ++j) {
                for (int r = 0; r < 4; ++r) h[j][r] *= PK ? gl[j][r] : eL;
                PolicyH::mma(h[j], ldKT(KG, j, 0), vb0);
            }
            const F yb1 = pack(y[2], y[3]);
            for (int it = 2; it < 4; ++it) PolicyH::mma(vn[it], ldA(Tc, offT[1] + it * 16 * 128), yb1);
            if (OUT && a.vnew) {
                // v_new of this wave's output rows (the partner stores the other half)
                for (int j = 0; j < 2; ++j) {
                    const int it = 2 * kq + j;
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * it + 4 * G + r;
                        if (i < len) a.vnew[((t0 + i) * H + head) * DV + col] = vn[it][r];
                    }
                }
            }
            for (int it = 2; it < 4; ++it)
                for (int r = 0; r < 4; ++r) vp[it][r] = PK ? vn[it][r] : vn[it][r] * cpf[it][r];
            const F vb1 = pack(vp[2], vp[3]);
            for (int j = 0; j < 4; ++j) PolicyH::mma(h[j], ldKT(KG, j, 1), vb1);
            // ---- output rows of this wave's half: scale (b^G (q h) + P v_new)
            if (OUT) {
                const F nb0 = pack(vn[0], vn[1]), nb1 = pack(vn[2], vn[3]);
                for (int j = 0; j < 2; ++j) {
                    const int it = 2 * kq + j;
                    f32x4 qh = {0.f, 0.f, 0.f, 0.f};
                    for (int s2 = 0; s2 < 4; ++s2) PolicyH::mma(qh, ldA(Q, offA[s2] + it * 16 * 256), hb[s2]);
                    f32x4 o;
                    if (PK) {
                        o = qh;                              // per key: q b^G is prepared
                    } else {
                        const f32x4 bq = *reinterpret_cast<const f32x4*>(&cf[CS_BQ + 16 * G + 4 * it]);
                        for (int r = 0; r < 4; ++r) o[r] = bq[r] * qh[r];
                    }
                    PolicyH::mma(o, ldA(Pc, offT[0] + it * 16 * 128), nb0);
                    if (kq == 1) PolicyH::mma(o, ldA(Pc, offT[1] + it * 16 * 128), nb1);
                    if (OXS) {
                        for (int r = 0; r < 4; ++r) ox[OXS ? tb : 0][(16 * it + 4 * G + r) * OXP + 16 * cg + n] = a.scale * o[r];
                    } else {
                        // per key: stored from here, non-temporal; rows past the
                        // chunk end fall outside the buffer range and are dropped
                        const int64_t rb = ((t0 + 16 * it) * H + head) * DV + vc0 + 16 * cg;   // wave-uniform
                        const uint32_t nrow = (uint32_t)max(len - 16 * it, 0);
                        for (int r = 0; r < 4; ++r) {
                            const uint32_t off = (uint32_t)(4 * G + r) * tokstride + n;
                            if (OBF) {
                                const rsrc_t ro = make_rsrc(reinterpret_cast<bf16*>(a.o) + rb, nrow * tokstride * 2);
                                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16)(a.scale * o[r])), ro, off * 2, 0, CP_NT);
                            } else {
                                const rsrc_t ro = make_rsrc(reinterpret_cast<float*>(a.o) + rb, nrow * tokstride * 4);
                                __builtin_amdgcn_raw_buffer_store_b32(f2u(a.scale * o[r]), ro, off * 4, 0, CP_NT);
                            }
                        }
                    }
                }
            }
            // after the output (q h uses the entry state): publish this wave's half of the next state operand
            for (int j2 = 0; j2 < 2; ++j2) {
                hb[2 * kq + j2] = pack_state(h[2 * j2], h[2 * j2 + 1]);
                hx[tq ^ 1][wv][j2][lane] = hb[2 * kq + j2].v;
            }
            lds_barrier();                          // chunk c consumed, chunk c+1 and the state operand published
        }
        // ---- results
        for (int j = 0; j < 4; ++j)
            for (int r = 0; r < 4; ++r) {
                const int key = 64 * kq + 16 * j + 4 * G + r;
                if (SUMMARY) {
                    if (mcols) { if (a.M) a.M[(uh * DK + key) * DK + col] = h[j][r]; }
                    else if (a.S_ext) a.S_ext[(uh * DK + key) * DV + col] = h[j][r];
                } else if (a.hfinal) {
                    a.hfinal[(uh * DK + key) * DV + col] = h[j][r];
                }
            }
    };
    if (wv < 4) {
        // ======================= compute waves
        if (wv >> 1) compute(std::integral_constant<int, 1>{});
        else compute(std::integral_constant<int, 0>{});
    } else {
        // ======================= streaming waves
        // Streaming wave 4 + r takes token rows 16r .. 16r+15 of every tile
        // (k and q rows, T, P, v), wave 4 also the coefficient block;
        // instantiated per r so that every register index is static.
        auto stream = [&](auto role_c) {
            constexpr int role = decltype(role_c)::value;
            const uint32_t rowb = tokstride * 2;         // bytes between token rows of k, q, v (bf16)
            // k / q rows: lane (row 8i + l/8, s = (l%8)/2, m = l%2) loads the
            // 16-byte pieces at keys 32s + 8m and 32s + 16 + 8m, which make up
            // operand granules 4s + 2m and 4s + 2m + 1 (i = 2 role, 2 role + 1)
            const int rl = lane >> 3, s = (lane & 7) >> 1, m = lane & 1;
            // [0..3] k, [4..7] q, [8..9] T, [10..11] P, [12] v, [13] coefficients,
            // per key [14..17] k b^{G_L - G}
            struct Set { u32x4 x[PK ? 18 : 14]; };
            auto load = [&](int c_, Set& d) {
                const int c = __builtin_amdgcn_readfirstlane(c_);
                const int len = chunk_len(c);
                const int64_t t0 = ui.start + (int64_t)c * BT;
                const int64_t ch = (int64_t)(ui.cbase + c) * H + head;
                const uint32_t span = len > 0 ? (uint32_t)(len - 1) * rowb + DK * 2 : 0;
                if (!PK) {
#pragma unroll
                    for (int kq = 0; kq < (OUT ? 2 : 1); ++kq) {
                        const rsrc_t rx = make_rsrc(reinterpret_cast<const bf16*>(kq ? a.q : a.k) + (t0 * H + head) * DK, span);
#pragma unroll
                        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                            for (int p = 0; p < 2; ++p)
                                d.x[4 * kq + 2 * ii + p] = __builtin_amdgcn_raw_buffer_load_b128(
                                    rx, (8 * (2 * role + ii) + rl) * rowb + (32 * s + 16 * p + 8 * m) * 2, 0, 0);
                    }
                } else {
                    // the prepared gated tiles (fp16, op_pos order, 256-byte rows):
                    // lane (row 8i + l/8) takes granules 2 (l%8) and 2 (l%8) + 1
#pragma unroll
                    for (int t3 = 0; t3 < 3; ++t3) {
                        if (t3 == 1 && !OUT) continue;
                        const void* src = t3 == 0 ? a.ws.kd : (t3 == 1 ? a.ws.qg : a.ws.kg);
                        const rsrc_t rx = make_rsrc(reinterpret_cast<const f16*>(src) + ch * (BT * DK), BT * DK * 2);
                        const int xb = t3 == 0 ? 0 : (t3 == 1 ? 4 : 14);
#pragma unroll
                        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                            for (int p = 0; p < 2; ++p)
                                d.x[xb + 2 * ii + p] = __builtin_amdgcn_raw_buffer_load_b128(
                                    rx, (8 * (2 * role + ii) + rl) * 256 + 16 * (2 * (lane & 7) + p), 0, 0);
                    }
                }
#pragma unroll
                for (int tp = 0; tp < (OUT ? 2 : 1); ++tp) {
                    const rsrc_t rt = make_rsrc(reinterpret_cast<const f16*>(tp ? a.ws.P : a.ws.Tm) + ch * (BT * BT), BT * BT * 2);
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        // rows 0..31 use operand positions 0..31 only: the pieces
                        // at 32..63 (zero blocks, never written) are out of range
                        const uint32_t off = (8 * (2 * role + ii) + (lane >> 3)) * 128 + 16 * (lane & 7);
                        d.x[8 + 2 * tp + ii] = __builtin_amdgcn_raw_buffer_load_b128(
                            rt, role < 2 && (lane & 7) >= 4 ? 0x40000000u : off, 0, 0);
                    }
                }
                // v rows 16 role + l/4, 16-byte piece l%4 of the tile's 32 columns
                const rsrc_t rv = make_rsrc(reinterpret_cast<const bf16*>(a.v) + (t0 * H + head) * DV + vc0,
                                            mcols ? 0u : (uint32_t)len * rowb);
                d.x[12] = __builtin_amdgcn_raw_buffer_load_b128(rv, (16 * role + (lane >> 2)) * rowb + 16 * (lane & 3), 0, 0);
                if (role == 0) {
                    const rsrc_t rc = make_rsrc(reinterpret_cast<const char*>(a.ws.cfh) + ch * CFS, CFS);
                    // used: scalar gate float 0 and floats 64..255; per key the
                    // beta row (bytes 384..511) and the fp32 b^{G_L} (bytes 512..1023)
                    const bool used = PK ? lane >= 24 : (lane == 0 || lane >= 16);
                    d.x[13] = __builtin_amdgcn_raw_buffer_load_b128(rc, used ? 16u * lane : 0x40000000u, 0, 0);
                }
            };
            auto store = [&](const Set& d, int buf) {
                if (PK) {
                    // granule g of row r at g ^ swzk(r), odd granules with swapped halves
#pragma unroll
                    for (int t3 = 0; t3 < 3; ++t3) {
                        if (t3 == 1 && !OUT) continue;
                        char* dx = reinterpret_cast<char*>(t3 == 0 ? kt[buf] : (t3 == 1 ? qt[OUT ? buf : 0] : gt[PK ? buf : 0]));
                        const int xb = t3 == 0 ? 0 : (t3 == 1 ? 4 : 14);
#pragma unroll
                        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                            for (int p = 0; p < 2; ++p) {
                                const int row = 8 * (2 * role + ii) + rl, g = 2 * (lane & 7) + p;
                                const u32x4 w = d.x[xb + 2 * ii + p];
                                *reinterpret_cast<u32x4*>(dx + row * 256 + ((g ^ swzk(row)) << 4)) =
                                    p ? u32x4{w[2], w[3], w[0], w[1]} : w;
                            }
                    }
                }
#pragma unroll
                for (int kq = 0; kq < (OUT && !PK ? 2 : (PK ? 0 : 1)); ++kq) {
                    char* dx = reinterpret_cast<char*>(kq ? qt[OUT ? buf : 0] : kt[buf]);
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int row = 8 * (2 * role + ii) + rl, g0 = 4 * s + 2 * m;
                        const u32x4 A = bf16x8_to_f16x8(d.x[4 * kq + 2 * ii]), B = bf16x8_to_f16x8(d.x[4 * kq + 2 * ii + 1]);
                        *reinterpret_cast<u32x4*>(dx + row * 256 + ((g0 ^ swzk(row)) << 4)) = u32x4{A[0], A[1], B[0], B[1]};
                        *reinterpret_cast<u32x4*>(dx + row * 256 + (((g0 + 1) ^ swzk(row)) << 4)) = u32x4{B[2], B[3], A[2], A[3]};
                    }
                }
#pragma unroll
                for (int tp = 0; tp < (OUT ? 2 : 1); ++tp) {
                    char* dt = reinterpret_cast<char*>(tp ? Pt[OUT ? buf : 0] : Tt[buf]);
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int row = 8 * (2 * role + ii) + (lane >> 3);
                        *reinterpret_cast<u32x4*>(dt + row * 128 + (((lane & 7) ^ swz8(row)) << 4)) = d.x[8 + 2 * tp + ii];
                    }
                }
                *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(vt[buf]) + role * 1024 + 16 * lane) = d.x[12];
                if (role == 0) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(cb[buf]) + 16 * lane) = d.x[13];
            };
            // output rows 16 role .. +15 of chunk co from the LDS tile: copy i
            // covers rows 16 role + 8i .. +7, 8 lanes (16 bytes each) per row
            auto store_out = [&](int co_) {
                const int co = __builtin_amdgcn_readfirstlane(co_);
                const int len = chunk_len(co);
                const int64_t rb = ((ui.start + (int64_t)co * BT + 16 * role) * H + head) * DV + vc0;
                const uint32_t nrow = (uint32_t)max(len - 16 * role, 0);
                const float* src = ox[OXS ? (co & 1) : 0];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int rr = 8 * i + (lane >> 3), c4 = 4 * (lane & 7);
                    const f32x4 x = *reinterpret_cast<const f32x4*>(&src[(16 * role + rr) * OXP + c4]);
                    const uint32_t off = (uint32_t)rr * tokstride + c4;
                    if (OBF) {
                        const rsrc_t ro = make_rsrc(reinterpret_cast<bf16*>(a.o) + rb, nrow * tokstride * 2);
                        const u32x2 w = {(uint32_t)__builtin_bit_cast(uint16_t, (bf16)x[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)x[1]) << 16),
                                         (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)x[3]) << 16)};
                        __builtin_amdgcn_raw_buffer_store_b64(w, ro, off * 2, 0, CP_NT);
                    } else {
                        const rsrc_t ro = make_rsrc(reinterpret_cast<float*>(a.o) + rb, nrow * tokstride * 4);
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), ro, off * 4, 0, CP_NT);
                    }
                }
            };
            // two register sets: even chunks in sa, odd chunks in sb
            Set sa, sb;
            if (nch > 0) {
                load(0, sa);
                load(min(1, nch - 1), sb);
                store(sa, 0);
            }
            lds_barrier();
            // Step c: the loads of chunk c + 2 into the set that held chunk
            // c, the output of chunk c - 1 (left in LDS during step c - 1),
            // then chunk c + 1 (loaded a step ago) into the LDS buffers that
            // chunk c - 1 released. The loop is unrolled by two so that each
            // set keeps its registers. Chunk indices are clamped, so the last
            // steps repeat the last chunk.
            for (int c = 0; c < nch; c += 2) {
                load(min(c + 2, nch - 1), sa);
                if (OXS && c > 0) store_out(c - 1);
                store(sb, 1);
                lds_barrier();
                if (c + 1 < nch) {
                    load(min(c + 3, nch - 1), sb);
                    if (OXS) store_out(c);
                    store(sa, 0);
                    lds_barrier();
                }
            }
            if (OXS && nch > 0) store_out(nch - 1);
        };
        if (wv == 4) stream(std::integral_constant<int, 0>{});
        else if (wv == 5) stream(std::integral_constant<int, 1>{});
        else if (wv == 6) stream(std::integral_constant<int, 2>{});
        else stream(std::integral_constant<int, 3>{});
    }
}

// ------------------------------------------------------------------ merge
constexpr int MC = 8;         // state columns per merge workgroup
constexpr int MLD = DK + 4;   // LDS row stride of M (16-byte rows, conflict-free column reads)

// One workgroup per (b, head, 8 state columns): S = M_s S + S_ext[s] over the
// segments in order. M_s (64 KiB) arrives as 16-byte loads, and the next
// segment's M and S_ext are in flight during the current product.
__global__ __launch_bounds__(256) void merge_kernel(int H, int n_seg, const float* S_ext, const float* M,
                                                     const float* S0, float* S_init, float* S_final) {
    __shared__ __attribute__((aligned(16))) float Ms[DK * MLD];
    __shared__ float Sc[DK * MC];
    const int tid = threadIdx.x, c = tid % MC, rbase = tid / MC;   // rows rbase + 32 i
    const int col0 = blockIdx.x * MC, bh = blockIdx.y, b = bh / H, head = bh % H;
    for (int i = 0; i < 4; ++i) {
        const int r = rbase + 32 * i;
        Sc[r * MC + c] = S0 ? S0[((int64_t)bh * DK + r) * DV + col0 + c] : 0.0f;
    }
    f32x4 mr[16];
    float er[4];
    auto load = [&](int s) {
        const int64_t us = ((int64_t)b * n_seg + s) * H + head;
        const f32x4* src = reinterpret_cast<const f32x4*>(M + us * DK * DK);
#pragma unroll
        for (int j = 0; j < 16; ++j) mr[j] = src[tid + 256 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i) er[i] = S_ext[(us * DK + rbase + 32 * i) * DV + col0 + c];
    };
    if (n_seg > 0) load(0);
    for (int s = 0; s < n_seg; ++s) {
        const int64_t us = ((int64_t)b * n_seg + s) * H + head;
        __syncthreads();                          // the previous product has read Ms and written Sc
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + 32 * i;
            S_init[(us * DK + r) * DV + col0 + c] = Sc[r * MC + c];
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = 4 * (tid + 256 * j);
            *reinterpret_cast<f32x4*>(&Ms[(e / DK) * MLD + e % DK]) = mr[j];
        }
        float acc[4];
        for (int i = 0; i < 4; ++i) acc[i] = er[i];
        if (s + 1 < n_seg) load(s + 1);
        __syncthreads();
        for (int m = 0; m < DK; ++m) {
            const float sv = Sc[m * MC + c];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += Ms[(rbase + 32 * i) * MLD + m] * sv;
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

// The adjoint of the merge, over the segments in reverse: with G_n the
// gradient at the end of the last segment (zero when dS_final is NULL),
// dS_exit[s] = G_{s+1} and G_s = M_s^T G_{s+1} + dS_ext[s]; dS0 = G_0. One
// workgroup per (b, head, 8 state columns). While G is known to be zero (no
// final-state gradient yet) the map is not read; M_0 is read only for dS0.
__global__ __launch_bounds__(256) void merge_adjoint_kernel(int H, int n_seg, const float* dS_ext, const float* M,
                                                             const float* dS_final, float* dS_exit, float* dS0) {
    __shared__ __attribute__((aligned(16))) float Ms[DK * MLD];
    __shared__ float Sc[DK * MC];
    const int tid = threadIdx.x, c = tid % MC, rbase = tid / MC;   // rows rbase + 32 i
    const int col0 = blockIdx.x * MC, bh = blockIdx.y, b = bh / H, head = bh % H;
    for (int i = 0; i < 4; ++i) {
        const int r = rbase + 32 * i;
        Sc[r * MC + c] = dS_final ? dS_final[((int64_t)bh * DK + r) * DV + col0 + c] : 0.0f;
    }
    bool zero = dS_final == nullptr;
    for (int s = n_seg - 1; s >= 0; --s) {
        const int64_t us = ((int64_t)b * n_seg + s) * H + head;
        __syncthreads();                          // Sc written, the previous product done with Ms
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + 32 * i;
            dS_exit[(us * DK + r) * DV + col0 + c] = Sc[r * MC + c];
        }
        if (s == 0 && !dS0) break;
        float acc[4];
        for (int i = 0; i < 4; ++i) acc[i] = dS_ext[(us * DK + rbase + 32 * i) * DV + col0 + c];
        if (!zero) {
            const f32x4* src = reinterpret_cast<const f32x4*>(M + us * DK * DK);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int e = 4 * (tid + 256 * j);
                *reinterpret_cast<f32x4*>(&Ms[(e / DK) * MLD + e % DK]) = src[tid + 256 * j];
            }
            __syncthreads();
            // (M^T G)[i][c] = sum_m M[m][i] G[m][c]
            for (int m = 0; m < DK; ++m) {
                const float gv = Sc[m * MC + c];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += Ms[m * MLD + rbase + 32 * i] * gv;
            }
        }
        __syncthreads();
        for (int i = 0; i < 4; ++i) Sc[(rbase + 32 * i) * MC + c] = acc[i];
        zero = false;
    }
    __syncthreads();
    if (dS0)
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + 32 * i;
            dS0[((int64_t)bh * DK + r) * DV + col0 + c] = Sc[r * MC + c];
        }
}

hipError_t launch_merge_adjoint(int B, int H, int n_seg, const float* dS_ext, const float* M,
                                const float* dS_final, float* dS_exit, float* dS0, hipStream_t s) {
    if (B * H == 0) return hipSuccess;
    dim3 grid(DV / MC, B * H);
    hipLaunchKernelGGL(merge_adjoint_kernel, grid, dim3(256), 0, s, H, n_seg, dS_ext, M, dS_final, dS_exit, dS0);
    return hipGetLastError();
}

// Pieces of a sequence split over packed documents, in token order: piece p
// enters with its document's initial state (zero when S0 is NULL) when it
// starts the document, else with the exit state of piece p - 1,
// M_{p-1} S_in[p-1] + S_ext[p-1]. Documents are independent: one workgroup
// per (8 state columns, head, document) walks that document's pieces, found
// by binary search in the non-decreasing piece_doc. While the entry state is
// known to be zero (the document's first piece without S0) the map is not
// read, so its summary may be skipped; the next map and S_ext are in flight
// during the current product.
__global__ __launch_bounds__(256) void merge_pieces_kernel(int H, int n_pieces, const int32_t* piece_doc,
                                                            const float* S_ext, const float* M, const float* S0,
                                                            float* S_in) {
    __shared__ __attribute__((aligned(16))) float Ms[DK * MLD];
    __shared__ float Sc[DK * MC];
    const int tid = threadIdx.x, c = tid % MC, rbase = tid / MC;   // rows rbase + 32 i
    const int col0 = (blockIdx.x % (DV / MC)) * MC, doc = blockIdx.x / (DV / MC), head = blockIdx.y;
    auto lower = [&](int d) {   // first piece whose document is >= d
        int lo = 0, hi = n_pieces;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (__builtin_amdgcn_readfirstlane(piece_doc[mid]) < d) lo = mid + 1;
            else hi = mid;
        }
        return lo;
    };
    const int p0 = lower(doc), p1 = lower(doc + 1);
    if (p0 >= p1) return;
    for (int i = 0; i < 4; ++i) {
        const int r = rbase + 32 * i;
        Sc[r * MC + c] = S0 ? S0[(((int64_t)doc * H + head) * DK + r) * DV + col0 + c] : 0.0f;
    }
    f32x4 mr[16];
    float er[4];
    auto load = [&](int p, bool with_map) {   // summary of piece p
        const int64_t ph = (int64_t)p * H + head;
        if (with_map) {
            const f32x4* src = reinterpret_cast<const f32x4*>(M + ph * DK * DK);
#pragma unroll
            for (int j = 0; j < 16; ++j) mr[j] = src[tid + 256 * j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) er[i] = S_ext[(ph * DK + rbase + 32 * i) * DV + col0 + c];
    };
    // the first piece's map is read only when the document has an entry state
    const bool map0 = S0 != nullptr;
    if (p0 + 1 < p1) load(p0, map0);
    for (int p = p0; p < p1; ++p) {
        __syncthreads();                          // the previous product has read Ms and written Sc
        for (int i = 0; i < 4; ++i) {
            const int r = rbase + 32 * i;
            S_in[(((int64_t)p * H + head) * DK + r) * DV + col0 + c] = Sc[r * MC + c];
        }
        if (p + 1 >= p1) break;
        const bool with_map = p > p0 || map0;
        if (with_map) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int e = 4 * (tid + 256 * j);
                *reinterpret_cast<f32x4*>(&Ms[(e / DK) * MLD + e % DK]) = mr[j];
            }
        }
        float acc[4];
        for (int i = 0; i < 4; ++i) acc[i] = er[i];
        if (p + 2 < p1) load(p + 1, true);
        __syncthreads();
        if (with_map)
            for (int m = 0; m < DK; ++m) {
                const float sv = Sc[m * MC + c];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += Ms[(rbase + 32 * i) * MLD + m] * sv;
            }
        __syncthreads();
        for (int i = 0; i < 4; ++i) Sc[(rbase + 32 * i) * MC + c] = acc[i];
    }
}

hipError_t launch_merge_pieces(int n_pieces, int n_docs, int H, const int32_t* piece_doc, const float* S_ext,
                               const float* M, const float* S0, float* S_in, hipStream_t s) {
    if (n_pieces == 0 || H == 0) return hipSuccess;
    dim3 grid((DV / MC) * n_docs, H);
    hipLaunchKernelGGL(merge_pieces_kernel, grid, dim3(256), 0, s, H, n_pieces, piece_doc, S_ext, M, S0, S_in);
    return hipGetLastError();
}

// ------------------------------------------------------------------ unit order
// Units of unequal length (packed documents, ragged segments) run their state
// passes longest first: workgroups are dispatched in grid order, so a long
// unit that starts last would stretch the tail of the pass. The rank of unit
// u is the number of units with more chunks, or as many chunks and a smaller
// index (a permutation); order[rank] = u.
constexpr int ORD_T = 1024;

__global__ __launch_bounds__(ORD_T) void unit_order_kernel(UnitMap um, int32_t* order) {
    __shared__ int32_t nch[ORD_T];
    const int n = um.n_units, tid = threadIdx.x;
    for (int u0 = 0; u0 < n; u0 += ORD_T) {
        const int u = u0 + tid;
        const int mine = u < n ? unit_info(um, u).nch : 0;
        int rank = 0;
        for (int v0 = 0; v0 < n; v0 += ORD_T) {
            __syncthreads();
            nch[tid] = v0 + tid < n ? unit_info(um, v0 + tid).nch : -1;
            __syncthreads();
            const int m = min(ORD_T, n - v0);
            for (int j = 0; j < m; ++j) {
                const int x = nch[j];
                rank += (x > mine) || (x == mine && v0 + j < u);
            }
        }
        if (u < n) order[rank] = u;
    }
}

// ------------------------------------------------------------------ launchers
// dynamic LDS that keeps a workgroup of `prep` off a compute unit that holds
// one of `state` (0 when the two cannot share one anyway)
static size_t lds_exclusion_pad(const void* prep, const void* state) {
    int dev = 0, lds_cu = 0;
    hipFuncAttributes fp, fs;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        hipFuncGetAttributes(&fp, prep) != hipSuccess || hipFuncGetAttributes(&fs, state) != hipSuccess)
        return 0;
    const long free_lds = (long)lds_cu - (long)fs.sharedSizeBytes;
    const long need = free_lds - (long)fp.sharedSizeBytes + 1024;
    // at most four workgroups per compute unit, so that the preparation
    // draws its bandwidth over the state pass's whole run instead of in
    // bursts that lengthen the state pass's loads
    const long quarter = (long)lds_cu / 4 - (long)fp.sharedSizeBytes;
    const long pad = need > quarter ? need : quarter;
    return pad > 0 ? (size_t)pad : 0;
}

hipError_t launch_prep(const Problem& p, const Workspace& ws, const void* k, const void* q,
                       const float* g, const void* beta, const PrepSlots& sl, hipStream_t s, bool off_state_cus) {
    if (p.um.n_chunks == 0) return hipSuccess;
    PrepArgs a;
    a.um = p.um; a.H = p.H; a.k = k; a.q = q; a.g = g; a.beta = beta; a.use_exp2 = p.use_exp2;
    a.ws = ws; a.g_cumsum = sl.g_cumsum; a.A = sl.A;
    a.qk_norm = p.qk_norm; a.beta_sig = p.beta_sig;
    a.q_hat = sl.q_hat; a.k_hat = sl.k_hat; a.q_rstd = sl.q_rstd; a.k_rstd = sl.k_rstd; a.beta_eff = sl.beta_eff;
    dim3 grid(p.um.n_chunks, p.H), block(256);
    const bool xf = a.qk_norm || a.beta_sig || a.q_hat || a.k_hat || a.q_rstd || a.k_rstd || a.beta_eff;
    if (p.dtype == 1) {
        if (p.per_key) {
            if (xf) hipLaunchKernelGGL(prep_kernel_pk<true>, grid, block, 0, s, a);
            else hipLaunchKernelGGL(prep_kernel_pk<false>, grid, block, 0, s, a);
        } else {
            const void* fn = xf ? reinterpret_cast<const void*>(prep_kernel_h<true>)
                                : reinterpret_cast<const void*>(prep_kernel_h<false>);
            const size_t pad = off_state_cus
                                   ? lds_exclusion_pad(fn, reinterpret_cast<const void*>(state_kernel_ks<false, false, false>))
                                   : 0;
            if (xf) hipLaunchKernelGGL(prep_kernel_h<true>, dim3(p.H * p.um.n_chunks), dim3(64), pad, s, a);
            else hipLaunchKernelGGL(prep_kernel_h<false>, dim3(p.H * p.um.n_chunks), dim3(64), pad, s, a);
        }
    } else {
        if (p.per_key) hipLaunchKernelGGL((prep_kernel<PolicyF, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((prep_kernel<PolicyF, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

// The preparation the backward reads: T, P and, for the scalar gate, the
// gate rows; per key, the gated q and k tiles and G_last. Natural order, fp32
// (T and P fp16 with bf16 inputs and a scalar gate).
hipError_t launch_prep_bwd(const Problem& p, const Workspace& ws, const void* k, const void* q, const float* g,
                           const void* beta, hipStream_t s) {
    if (p.um.n_chunks == 0) return hipSuccess;
    PrepArgs a;
    a.um = p.um; a.H = p.H; a.k = k; a.q = q; a.g = g; a.beta = beta; a.use_exp2 = p.use_exp2;
    a.ws = ws; a.g_cumsum = nullptr; a.A = nullptr;
    a.qk_norm = 0; a.beta_sig = 0;
    a.q_hat = nullptr; a.k_hat = nullptr; a.q_rstd = nullptr; a.k_rstd = nullptr; a.beta_eff = nullptr;
    dim3 grid(p.um.n_chunks, p.H), block(256);
    if (p.per_key) {
        if (p.dtype == 1) hipLaunchKernelGGL(prep_kernel_pkb, grid, block, 0, s, a);
        else hipLaunchKernelGGL((prep_kernel<PolicyF, true>), grid, block, 0, s, a);
    } else {
        if (p.dtype == 1) hipLaunchKernelGGL((prep_kernel_h<false, true>), dim3(p.H * p.um.n_chunks), dim3(64), 0, s, a);
        else hipLaunchKernelGGL((prep_kernel<PolicyF, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <class P, bool PK>
static void launch_state_t(bool summary, StateArgs a, int want_ext, int want_M, hipStream_t s) {
    if (summary) {
        a.tile0 = want_ext ? 0 : DV / BV;
        a.ntiles = (want_ext ? DV / BV : 0) + (want_M ? DK / BV : 0);
    } else {
        a.tile0 = 0;
        a.ntiles = DV / BV;
    }
    if (a.n_pairs == 0 || a.ntiles == 0) return;
    const int groups = (a.n_pairs + 7) / 8;
    dim3 grid(8 * a.ntiles * groups), block(ST);
    if (summary) hipLaunchKernelGGL((state_kernel<P, PK, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((state_kernel<P, PK, false>), grid, block, 0, s, a);
}

template <bool PK>
static void launch_state_h(bool summary, StateArgs a, int want_ext, int want_M, hipStream_t s) {
    if (summary) {
        a.tile0 = want_ext ? 0 : DV / BV;
        a.ntiles = (want_ext ? DV / BV : 0) + (want_M ? DK / BV : 0);
    } else {
        a.tile0 = 0;
        a.ntiles = DV / BV;
    }
    if (a.n_pairs == 0 || a.ntiles == 0) return;
    const int groups = (a.n_pairs + 7) / 8;
    dim3 grid(8 * a.ntiles * groups);
    if (summary) hipLaunchKernelGGL((state_kernel_ks<true, false, PK>), grid, dim3(KST), 0, s, a);
    else if (a.o_bf16) hipLaunchKernelGGL((state_kernel_ks<false, true, PK>), grid, dim3(KST), 0, s, a);
    else hipLaunchKernelGGL((state_kernel_ks<false, false, PK>), grid, dim3(KST), 0, s, a);
}

hipError_t launch_state(const Problem& p, const Workspace& ws, const void* q, const void* k,
                        const void* v, const void* beta, const float* h0, void* o, float* hfinal,
                        float* hslot, float* vnew_slot, int summary, int want_ext, int want_M, float* S_ext,
                        float* M, const int32_t* units_sel, int n_sel, hipStream_t s) {
    StateArgs a;
    a.vnew = summary ? nullptr : vnew_slot;
    a.beta_sig = p.beta_sig;
    a.um = p.um; a.H = p.H; a.q = q; a.k = k; a.v = v; a.beta = beta; a.ws = ws;
    a.h0 = h0; a.o = o; a.o_bf16 = p.o_dtype == 1; a.hfinal = hfinal; a.hslot = hslot;
    a.scale = p.scale; a.use_exp2 = p.use_exp2;
    a.n_pairs = p.um.n_units * p.H;
    a.S_ext = S_ext; a.M = M;
    a.ntiles = 0; a.tile0 = 0;
    a.order = nullptr;
    if (units_sel) {
        // only the selected units, in the caller's order
        a.order = units_sel;
        a.n_pairs = n_sel * p.H;
    } else if (ws.order && a.n_pairs > 0) {
        hipLaunchKernelGGL(unit_order_kernel, dim3(1), dim3(ORD_T), 0, s, p.um, ws.order);
        a.order = ws.order;
    }
    if (p.dtype == 1) {
        if (p.per_key) launch_state_h<true>(summary, a, want_ext, want_M, s);
        else launch_state_h<false>(summary, a, want_ext, want_M, s);
    } else {
        if (p.per_key) launch_state_t<PolicyF, true>(summary, a, want_ext, want_M, s);
        else launch_state_t<PolicyF, false>(summary, a, want_ext, want_M, s);
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
