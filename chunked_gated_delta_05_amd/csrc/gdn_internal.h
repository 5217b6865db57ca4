// Internal interface between the host API (gdn_host.cpp) and the HIP kernels
// (gdn_kernels.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "gdn.h"

namespace gdn {

constexpr int BT = 64;    // tokens per chunk
constexpr int DK = 128;   // key width
constexpr int DV = 128;   // value width
constexpr int BV = 32;    // value columns per state-pass workgroup
constexpr int CFB = 1024; // per-(chunk, head) coefficient block of the per-key fp16 state pass (bytes)
constexpr int CFS = 1024; // the same block of the scalar-gate fp16 state pass (bytes)
constexpr int GAMR = 5;       // fp32 scalar-gate rows per (chunk, head) in Workspace::gam
constexpr int ORD_MAX = 2048;  // packed units beyond this count keep their natural launch order

// Where every chunk of every unit lives on the flat token axis.
struct UnitMap {
    int32_t n_units;             // number of units (B when dense)
    int32_t dense;               // 1: unit b = tokens [t_base + b*row_stride, +T), no device metadata
    int32_t T;                   // dense unit length
    int32_t n_chunks;            // total chunks over all units
    int32_t nt_dense;            // chunks per dense unit
    int64_t total_tokens;
    int64_t row_stride;          // dense: tokens between unit starts (the row length)
    int64_t t_base;              // dense: token offset of unit 0 in its row (a piece of the rows)
    const int32_t* offsets;      // device [n_units + 1] (NULL when dense)
    const int32_t* chunk_offsets;// device [n_units + 1]
    const int32_t* chunk_indices;// device [n_chunks][2]
};

// Workspace regions, all device pointers inside the caller's workspace.
// Operand arrays hold fp16 for bf16 inputs and fp32 for fp32 inputs. With
// fp16 operands the 64-wide (T, P) and K-wide (the gated k and q forms)
// rows are stored in the state pass's operand order (op_pos in the kernels).
struct Workspace {
    void* Tm;        // operands [n_chunks][H][64][64]  T = (I + L)^{-1}
    void* P;         // operands [n_chunks][H][64][64]  decayed q.k, lower incl. diagonal
    float* gam;      // fp32 scalar gate only: [n_chunks][H][5][64]  G, b^G r_k, b^{G_last-G} r_k,
                     // b^{G_last}, b^G r_q (r: the reciprocal q / k norms, 1 without normalisation)
    // per-key gate only
    void* qg;        // operands [n_chunks][H][64][K]  q * b^G
    void* kd;        // operands [n_chunks][H][64][K]  k * b^G
    void* kg;        // operands [n_chunks][H][64][K]  k * b^{G_last - G}
    float* gamL;     // [n_chunks][H][K]  G at the chunk's last valid token
    // bf16 inputs only
    void* cfh;       // [n_chunks][H][1 KiB]  per-row coefficient block of the fp16 state pass
                     // (fp32 rows for the scalar gate, fp16 rows + fp32 gates per key)
    // packed units only
    int32_t* order;  // [n_units]  units in state-pass launch order (most chunks first)
};

struct Problem {
    int32_t H;
    int32_t dtype;      // 0 fp32, 1 bf16
    int32_t o_dtype;
    int32_t per_key;
    int32_t use_exp2;
    float scale;
    UnitMap um;
    int32_t reorder;    // packed units out of longest-first order: the state passes reorder them
    int32_t qk_norm;    // q and k L2-normalised in the kernels
    int32_t beta_sig;   // beta through a sigmoid in the kernels
};

// Optional per-token outputs of the chunk preparation (NULL: not written).
struct PrepSlots {
    float* g_cumsum;
    float* A;
    void* q_hat;        // input dtype [tokens][H][K]
    void* k_hat;
    float* q_rstd;      // [tokens][H]
    float* k_rstd;
    void* beta_eff;     // input dtype [tokens][H]
};

size_t workspace_bytes(const Problem& p, Workspace* ws, char* base);

// gdn_chunk_fwd itself; allow_pipeline = false keeps the single-pass
// workspace (the allocation-free entry point, whose scratch is sized for it)
gdn_status fwd_impl(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                    const void* beta, const float* initial_state, void* o, float* final_state, const gdn_slots* slots,
                    int32_t flags, void* workspace, size_t* workspace_bytes, hipStream_t stream, bool allow_pipeline);

// off_state_cus: the preparation runs beside a state pass of the same
// problem (the pieced forward); it then asks for enough LDS that its
// workgroups cannot share a compute unit with the state pass's
hipError_t launch_prep(const Problem& p, const Workspace& ws, const void* k, const void* q,
                       const float* g, const void* beta, const PrepSlots& slots, hipStream_t s,
                       bool off_state_cus = false);

// mode: 0 forward; 1 summary (S_ext and/or M), of the units in units_sel
// (device, n_sel entries) when given, else of all
hipError_t launch_state(const Problem& p, const Workspace& ws, const void* q, const void* k,
                        const void* v, const void* beta, const float* h0, void* o,
                        float* hfinal, float* hslot, float* vnew_slot, int summary, int want_ext, int want_M,
                        float* S_ext, float* M, const int32_t* units_sel, int n_sel, hipStream_t s);

hipError_t launch_merge_pieces(int n_pieces, int n_docs, int H, const int32_t* piece_doc, const float* S_ext,
                               const float* M, const float* S0, float* S_in, hipStream_t s);

hipError_t launch_merge(int B, int H, int n_seg, const float* S_ext, const float* M,
                        const float* S0, float* S_init, float* S_final, hipStream_t s);

hipError_t launch_merge_adjoint(int B, int H, int n_seg, const float* dS_ext, const float* M,
                                const float* dS_final, float* dS_exit, float* dS0, hipStream_t s);

// The chunk preparation the backward reads (T, P, gate rows; per key the
// gated tiles), natural order: fp32, or fp16 T and P for bf16 inputs with a
// scalar gate.
hipError_t launch_prep_bwd(const Problem& p, const Workspace& ws, const void* k, const void* q,
                           const float* g, const void* beta, hipStream_t s);

// The backward: the chunk preparation (skipped with reuse_prep: the workspace
// holds it), reverse state pass, per-chunk gradients (skipped with dh_only).
hipError_t launch_bwd(const Problem& p, const Workspace& ws, float* dH, float* dVN, const void* q,
                      const void* k, const void* v, const float* g, const void* beta, const float* h,
                      const void* dout, const float* dht, float* dq, float* dk, float* dv, float* dg,
                      float* dbeta, float* dh0, bool dh_only, bool reuse_prep, hipStream_t s);

// Host-only checks of a gdn_chunk_fwd call (descriptor, flags, pointers), and
// the workspace it needs; no HIP call.
gdn_status fwd_preflight(const gdn_desc* desc, const void* q, const void* k, const void* v,
                         const float* g, const void* beta, const void* o, int32_t flags, Problem* p,
                         size_t* workspace_need);

}  // namespace gdn
