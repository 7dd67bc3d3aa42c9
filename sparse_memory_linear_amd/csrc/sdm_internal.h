// Internal launch interface between the C ABI (sdm_api.hip) and the kernels.
// Not installed, not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

struct AddressArgs {
    const void* q[2];        // per branch: [B,H,T,2,dh]
    const void* K[2];        // per branch: [H,2,n,dh]
    int32_t* idx[2];         // [B,H,T,k]
    float* wt[2];
    float* score[2];         // optional
    int k[2];
    float* half_out;         // debug: [B,H,T,2,n]; when set only half-scores are written
    int64_t B, H, T;
    int n, dh;
    int nbranch;             // 1 or 2
    bool bf16;
    bool idw;                // inverse-distance half-scores instead of dot products
};
hipError_t launch_address(const AddressArgs& a, hipStream_t st);

// The output step fused into the scan's last pass (partial sums of the row
// partitions -> y -> RMS-Norm and output gate -> o): see sdm_scan_forward_gated.
struct GateArgs {
    const float* gamma;      // [H,dv]
    const void* g;           // [B,H,T,dv] gate pre-activation
    float* o;                // [B,H,T,dv]
    float eps;
    int64_t H;
    bool g_bf16;
};

struct ScanArgs {
    const int32_t* idx_w; const float* wt_w; int W;
    const int32_t* idx_r; const float* wt_r; int R;
    const float* alpha; const float* beta;
    const void* v; bool v_bf16;
    void* M; bool m_bf16;    // table elements: fp32, or bfloat16 (no pre-images then)
    float* y;
    int64_t NS;              // B*H streams
    int64_t T, N;
    int dv;
    int form;                // 0 = per-slot Eq. (4), 1 = Fig. 2 shared residual
    void* workspace;
    float* snap;             // optional [NS][T][W][dv]: pre-image of every write (training forward)
    int64_t max_tokens = 0;  // > 0: tokens per launch chunk at most this (a bounded workspace)
    // optional: the output step; where the scan sums row-partition partials it
    // runs in that pass (y is then stored only if y != nullptr), else the caller
    // runs the output gate on y
    const GateArgs* gate = nullptr;
};
// Whether launch_scan with a.gate set fuses the output step for these sizes
// (else y is stored and the caller applies the gate).
bool scan_fuses_gate(int64_t NS, int64_t T, int W, int R, int dv, bool m_bf16, int form);
// Chooses the kernel instance; returns false if no instance covers (W, R, dv).
bool scan_geometry(int64_t NS, int W, int R, int dv, bool m_bf16, int* slab, int* rec_bytes);
int64_t scan_workspace_bytes(int64_t NS, int64_t T, int W, int R, int dv);
// The most tokens per launch chunk (at most T) whose workspace fits in `bytes`
// for this table dtype and form; T itself when the call takes the short-call
// form (no workspace); 0 when not even one token fits.
int64_t scan_tokens_within(int64_t NS, int64_t T, int W, int R, int dv, bool m_bf16, int form, int64_t bytes);
hipError_t launch_scan(const ScanArgs& a, hipStream_t st);

struct BwdArgs {
    const int32_t* idx_w; const float* wt_w; int W;
    const int32_t* idx_r; const float* wt_r; int R;
    const float* alpha; const float* beta;
    const void* v; bool v_bf16;
    const float* snap;       // [NS][T][W][dv] from the training forward
    const float* dy;         // [NS][T][dv]
    float* M;                // in: state after token T-1; out: before token 0 (restored)
    float* dM;               // in: dL/dM after token T-1; out: dL/dM before token 0
    float* dv_out;           // [NS][T][dv]
    float* dalpha; float* dbeta;   // [NS][T]
    float* dwt_w; float* dwt_r;    // [NS][T][W], [NS][T][R]
    int64_t NS, T, N;
    int dv;
    int form;
    void* workspace;
};
int64_t scan_backward_workspace_bytes(int64_t NS, int64_t T, int W, int R, int dv);
bool scan_backward_geometry(int64_t NS, int W, int R, int dv);
hipError_t launch_scan_backward(const BwdArgs& a, hipStream_t st);
hipError_t launch_state_init_backward(const float* dM, float* dM0, int64_t B, int64_t per_seq, hipStream_t st);

hipError_t launch_state_init(const float* M0, void* M, bool m_bf16, int64_t B, int64_t per_seq, hipStream_t st);

struct GatesArgs {
    const void* x;           // [B,T,d]
    const void* Wa;          // [H,d]
    const void* Wb;          // [H,d]
    const float* bdt;        // [H]
    const float* A;          // [H]
    float* alpha; float* beta;  // [B,H,T]
    int64_t B, T;
    int d, H;
    bool bf16;
};
hipError_t launch_gates(const GatesArgs& a, hipStream_t st);

struct OutGateArgs {
    const float* y;          // [B,H,T,dv]
    const float* gamma;      // [H,dv]
    const void* g;           // [B,H,T,dv]
    float* o;                // [B,H,T,dv]
    float eps;
    int64_t rows, T, H;      // rows = B*H*T
    int dv, lg;
    bool g_bf16;
};
hipError_t launch_output_gate(OutGateArgs a, hipStream_t st);

// Lanes per row of the output step: a power of two covering the row's 16-byte
// pieces, at most 64 (the same in the plain and the fused kernel, so both add
// the squares in the same order).
__host__ __device__ inline int output_gate_lanes(int dv) {
    int lg = 1;
    while (lg < 64 && lg < dv / 4) lg <<= 1;
    return lg;
}
// The fused form holds a lane's pieces in registers: at most this many.
constexpr int GATE_FUSED_PIECES = 4;
// The partial sums of P row partitions of one launch chunk (Tc of TS tokens
// from t0) -> y (if y != nullptr) and the output step -> o.
struct YGateArgs {
    const float* yp;         // [P][NS][Tc][dv]
    float* y;                // [NS][TS][dv] or nullptr
    GateArgs gate;
    int P;
    int64_t NS, Tc, TS, t0;
    int dv;
};
hipError_t launch_ypart_gate(const YGateArgs& a, hipStream_t st);

}  // namespace sdm
