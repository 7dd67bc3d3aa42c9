// sdm_api.hip -- the C ABI (include/sdm.h): host-side validation and dispatch.
// Every check runs before any HIP call; a failing call writes nothing,
// launches nothing and records a thread-local message.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "sdm.h"
#include "sdm_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return SDM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_fail(hipError_t e, const char* what) {
    return fail(SDM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_address_sizes(int q_dtype, int k_dtype, int64_t B, int64_t H, int64_t T, int64_t n_sub,
                        int64_t dh) {
    if (q_dtype != SDM_F32 && q_dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "unknown q dtype %d", q_dtype);
    if (k_dtype != q_dtype) return fail(SDM_ERR_DTYPE, "subkey dtype %d differs from q dtype %d", k_dtype, q_dtype);
    if (B < 0 || H < 0 || T < 0) return fail(SDM_ERR_SHAPE, "negative B/H/T (%lld, %lld, %lld)",
                                             (long long)B, (long long)H, (long long)T);
    if (n_sub < 1 || dh < 1) return fail(SDM_ERR_SHAPE, "n_sub and dh must be >= 1");
    if (n_sub % 16 != 0 || n_sub > 512)
        return fail(SDM_ERR_UNSUPPORTED, "n_sub=%lld: kernels cover multiples of 16 up to 512", (long long)n_sub);
    const int64_t step = q_dtype == SDM_BF16 ? 32 : 8;
    if (dh % step != 0 || dh > 256)
        return fail(SDM_ERR_UNSUPPORTED, "dh=%lld: kernels cover multiples of %lld up to 256", (long long)dh,
                    (long long)step);
    const int64_t ntile = (B * T + 15) / 16;
    if (ntile * H > 0x7FFFFFFFll) return fail(SDM_ERR_UNSUPPORTED, "too many token tiles for one launch");
    // token numbers b * T + t are kept in 32 bits on the GPU
    if (B * T > 0xFFFFFFFFll) return fail(SDM_ERR_UNSUPPORTED, "B*T=%lld: at most 2^32 - 1 tokens per call",
                                          (long long)(B * T));
    return SDM_OK;
}

}  // namespace

extern "C" {

int sdm_abi_version(void) { return SDM_ABI_VERSION; }

const char* sdm_status_string(int s) {
    switch (s) {
        case SDM_OK: return "ok";
        case SDM_ERR_NULL: return "null pointer";
        case SDM_ERR_SHAPE: return "invalid shape";
        case SDM_ERR_DTYPE: return "invalid dtype or form";
        case SDM_ERR_ALIGN: return "pointer not 16-byte aligned";
        case SDM_ERR_UNSUPPORTED: return "unsupported size";
        case SDM_ERR_HIP: return "HIP error";
        case SDM_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

const char* sdm_last_error(void) { return g_err; }

static int address_impl(const char* fn, bool idw, const void* q_w, const void* q_r, int q_dtype,
                        const void* subkeys_w, const void* subkeys_r, int k_dtype, int64_t B, int64_t H, int64_t T,
                        int64_t n_sub, int64_t dh, int64_t W, int64_t R, int32_t* idx_w, float* wt_w,
                        int32_t* idx_r, float* wt_r, float* score_w, float* score_r, void* stream) {
    int rc = check_address_sizes(q_dtype, k_dtype, B, H, T, n_sub, dh);
    if (rc) return rc;
    const int64_t N = n_sub * n_sub;
    if (W < 1 || R < 1 || W > N || R > N)
        return fail(SDM_ERR_SHAPE, "W=%lld, R=%lld must lie in [1, N=%lld]", (long long)W, (long long)R,
                    (long long)N);
    if (W > 64 || R > 64) return fail(SDM_ERR_UNSUPPORTED, "W, R <= 64 on the GPU (W=%lld, R=%lld)",
                                      (long long)W, (long long)R);
    if (B == 0 || H == 0 || T == 0) return ok();  // empty tensors may have NULL data
    if (!q_w || !q_r || !subkeys_w || !subkeys_r || !idx_w || !wt_w || !idx_r || !wt_r)
        return fail(SDM_ERR_NULL, "%s: a required pointer is NULL", fn);
    const void* ptrs[] = {q_w, q_r, subkeys_w, subkeys_r, idx_w, wt_w, idx_r, wt_r};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SDM_ERR_ALIGN, "%s: pointer %p not 16-byte aligned", fn, p);
    if ((score_w && !aligned16(score_w)) || (score_r && !aligned16(score_r)))
        return fail(SDM_ERR_ALIGN, "%s: score pointer not 16-byte aligned", fn);
    sdm::AddressArgs a{};
    a.q[0] = q_w; a.q[1] = q_r;
    a.K[0] = subkeys_w; a.K[1] = subkeys_r;
    a.idx[0] = idx_w; a.idx[1] = idx_r;
    a.wt[0] = wt_w; a.wt[1] = wt_r;
    a.score[0] = score_w; a.score[1] = score_r;
    a.k[0] = (int)W; a.k[1] = (int)R;
    a.half_out = nullptr;
    a.B = B; a.H = H; a.T = T; a.n = (int)n_sub; a.dh = (int)dh;
    a.nbranch = 2;
    a.bf16 = q_dtype == SDM_BF16;
    a.idw = idw;
    hipError_t e = sdm::launch_address(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

static int half_scores_impl(const char* fn, bool idw, const void* q, int q_dtype, const void* subkeys, int k_dtype,
                            int64_t B, int64_t H, int64_t T, int64_t n_sub, int64_t dh, float* half, void* stream) {
    int rc = check_address_sizes(q_dtype, k_dtype, B, H, T, n_sub, dh);
    if (rc) return rc;
    if (B == 0 || H == 0 || T == 0) return ok();
    if (!q || !subkeys || !half) return fail(SDM_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned16(q) || !aligned16(subkeys) || !aligned16(half))
        return fail(SDM_ERR_ALIGN, "%s: pointer not 16-byte aligned", fn);
    sdm::AddressArgs a{};
    a.q[0] = q; a.K[0] = subkeys;
    a.k[0] = 1;
    a.half_out = half;
    a.B = B; a.H = H; a.T = T; a.n = (int)n_sub; a.dh = (int)dh;
    a.nbranch = 1;
    a.bf16 = q_dtype == SDM_BF16;
    a.idw = idw;
    hipError_t e = sdm::launch_address(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

int sdm_address(const void* q_w, const void* q_r, int q_dtype, const void* subkeys_w, const void* subkeys_r,
                int k_dtype, int64_t B, int64_t H, int64_t T, int64_t n_sub, int64_t dh, int64_t W, int64_t R,
                int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r, float* score_w, float* score_r,
                void* stream) {
    return address_impl("sdm_address", false, q_w, q_r, q_dtype, subkeys_w, subkeys_r, k_dtype, B, H, T, n_sub, dh,
                        W, R, idx_w, wt_w, idx_r, wt_r, score_w, score_r, stream);
}

int sdm_address_idw(const void* q_w, const void* q_r, int q_dtype, const void* subkeys_w, const void* subkeys_r,
                    int k_dtype, int64_t B, int64_t H, int64_t T, int64_t n_sub, int64_t dh, int64_t W, int64_t R,
                    int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r, float* score_w, float* score_r,
                    void* stream) {
    return address_impl("sdm_address_idw", true, q_w, q_r, q_dtype, subkeys_w, subkeys_r, k_dtype, B, H, T, n_sub,
                        dh, W, R, idx_w, wt_w, idx_r, wt_r, score_w, score_r, stream);
}

int sdm_debug_half_scores(const void* q, int q_dtype, const void* subkeys, int k_dtype, int64_t B, int64_t H,
                          int64_t T, int64_t n_sub, int64_t dh, float* half, void* stream) {
    return half_scores_impl("sdm_debug_half_scores", false, q, q_dtype, subkeys, k_dtype, B, H, T, n_sub, dh, half,
                            stream);
}

int sdm_debug_half_scores_idw(const void* q, int q_dtype, const void* subkeys, int k_dtype, int64_t B, int64_t H,
                              int64_t T, int64_t n_sub, int64_t dh, float* half, void* stream) {
    return half_scores_impl("sdm_debug_half_scores_idw", true, q, q_dtype, subkeys, k_dtype, B, H, T, n_sub, dh,
                            half, stream);
}

int sdm_state_init(const float* M0, void* M, int m_dtype, int64_t B, int64_t H, int64_t N, int64_t dv,
                   void* stream) {
    if (m_dtype != SDM_F32 && m_dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "unknown table dtype %d", m_dtype);
    if (B < 0 || H < 0 || N < 1 || dv < 1) return fail(SDM_ERR_SHAPE, "sdm_state_init: invalid sizes");
    if (dv % 4 != 0) return fail(SDM_ERR_UNSUPPORTED, "sdm_state_init: dv must be a multiple of 4");
    if (B == 0 || H == 0) return ok();
    if (!M0 || !M) return fail(SDM_ERR_NULL, "sdm_state_init: NULL pointer");
    if (!aligned16(M0) || !aligned16(M)) return fail(SDM_ERR_ALIGN, "sdm_state_init: pointer not 16-byte aligned");
    hipError_t e = sdm::launch_state_init(M0, M, m_dtype == SDM_BF16, B, H * N * dv,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sdm_state_init launch");
    return ok();
}

int64_t sdm_scan_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t W, int64_t R, int64_t dv) {
    if (B < 0 || H < 0 || T < 0 || W < 1 || R < 1 || W > 256 || R > 256 || dv < 4 || dv % 4) return -1;
    if (B == 0 || H == 0 || T == 0) return 0;
    return sdm::scan_workspace_bytes(B * H, T, (int)W, (int)R, (int)dv);
}

}  // extern "C"

namespace {

// Shared checks of the scan entry points (sizes, dtypes, pointers, alignment,
// workspace). 0 when the call may launch; NO_WORK when there is no work (the
// call succeeds and launches nothing); otherwise the status code.
constexpr int NO_WORK = -1;
int check_scan(const char* fn, const int32_t* idx_w, const float* wt_w, int64_t W, const int32_t* idx_r,
               const float* wt_r, int64_t R, const float* alpha, const float* beta, const void* v, int v_dtype,
               int64_t B, int64_t H, int64_t T, int64_t N, int64_t dv, int form, int m_dtype = SDM_F32) {
    if (v_dtype != SDM_F32 && v_dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "unknown v dtype %d", v_dtype);
    if (m_dtype != SDM_F32 && m_dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "unknown table dtype %d", m_dtype);
    if (form != SDM_DELTA_EQ4 && form != SDM_DELTA_FIG2) return fail(SDM_ERR_DTYPE, "unknown delta form %d", form);
    if (B < 0 || H < 0 || T < 0 || N < 1 || dv < 1) return fail(SDM_ERR_SHAPE, "%s: invalid sizes", fn);
    if (W < 1 || R < 1 || W > N || R > N)
        return fail(SDM_ERR_SHAPE, "W=%lld, R=%lld must lie in [1, N=%lld]", (long long)W, (long long)R,
                    (long long)N);
    if (W > 256 || R > 256) return fail(SDM_ERR_UNSUPPORTED, "W, R <= 256 on the GPU");
    if (N > (1 << 18)) return fail(SDM_ERR_UNSUPPORTED, "N=%lld: at most 2^18 slots", (long long)N);
    if (dv % 4 != 0) return fail(SDM_ERR_UNSUPPORTED, "dv=%lld must be a multiple of 4", (long long)dv);
    if (m_dtype == SDM_BF16 && dv % 8 != 0)
        return fail(SDM_ERR_UNSUPPORTED, "dv=%lld must be a multiple of 8 for a bf16 table", (long long)dv);
    if (N * dv * 4 >= (1ll << 31))
        return fail(SDM_ERR_UNSUPPORTED, "one stream's table (N*dv*4 = %lld bytes) must stay below 2 GiB",
                    (long long)(N * dv * 4));
    if (!sdm::scan_geometry(B * H > 0 ? B * H : 1, (int)W, (int)R, (int)dv, m_dtype == SDM_BF16, nullptr,
                            nullptr))
        return fail(SDM_ERR_UNSUPPORTED, "no scan kernel covers W=%lld, R=%lld, dv=%lld", (long long)W,
                    (long long)R, (long long)dv);
    if ((B * H + 7) / 8 * 8 * (dv / 4) > 0x7FFFFFFFll)
        return fail(SDM_ERR_UNSUPPORTED, "too many streams for one launch");
    if (B == 0 || H == 0 || T == 0) return NO_WORK;  // empty tensors may have NULL data
    if (!idx_w || !wt_w || !idx_r || !wt_r || !alpha || !beta || !v)
        return fail(SDM_ERR_NULL, "%s: a required pointer is NULL", fn);
    const void* ptrs[] = {idx_w, wt_w, idx_r, wt_r, alpha, beta, v};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SDM_ERR_ALIGN, "%s: pointer %p not 16-byte aligned", fn, p);
    return 0;
}

int check_buffers(const char* fn, std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs) {
        if (!p) return fail(SDM_ERR_NULL, "%s: a required pointer is NULL", fn);
        if (!aligned16(p)) return fail(SDM_ERR_ALIGN, "%s: pointer %p not 16-byte aligned", fn, p);
    }
    return 0;
}

int check_workspace(void* workspace, int64_t workspace_bytes, int64_t need) {
    if (!workspace || workspace_bytes < need)
        return fail(SDM_ERR_WORKSPACE, "workspace of %lld bytes needed, %lld given", (long long)need,
                    (long long)(workspace ? workspace_bytes : 0));
    if (!aligned16(workspace)) return fail(SDM_ERR_ALIGN, "workspace not 16-byte aligned");
    return 0;
}

int scan_forward_impl(const char* fn, const int32_t* idx_w, const float* wt_w, int64_t W, const int32_t* idx_r,
                      const float* wt_r, int64_t R, const float* alpha, const float* beta, const void* v,
                      int v_dtype, void* M, int m_dtype, float* y, float* snap, bool save, int64_t B, int64_t H,
                      int64_t T, int64_t N, int64_t dv, int form, void* workspace, int64_t workspace_bytes,
                      void* stream) {
    int rc = check_scan(fn, idx_w, wt_w, W, idx_r, wt_r, R, alpha, beta, v, v_dtype, B, H, T, N, dv, form,
                        m_dtype);
    if (rc == NO_WORK) return ok();
    if (rc) return rc;
    if ((rc = check_buffers(fn, {M, y}))) return rc;
    if (save && (rc = check_buffers(fn, {snap}))) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes,
                              sdm::scan_workspace_bytes(B * H, T, (int)W, (int)R, (int)dv))))
        return rc;
    sdm::ScanArgs a{};
    a.idx_w = idx_w; a.wt_w = wt_w; a.W = (int)W;
    a.idx_r = idx_r; a.wt_r = wt_r; a.R = (int)R;
    a.alpha = alpha; a.beta = beta;
    a.v = v; a.v_bf16 = v_dtype == SDM_BF16;
    a.M = M; a.m_bf16 = m_dtype == SDM_BF16; a.y = y;
    a.NS = B * H; a.T = T; a.N = N; a.dv = (int)dv;
    a.form = form;
    a.workspace = workspace;
    a.snap = save ? snap : nullptr;
    hipError_t e = sdm::launch_scan(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

}  // namespace

extern "C" {

int sdm_scan_forward(const int32_t* idx_w, const float* wt_w, int64_t W, const int32_t* idx_r, const float* wt_r,
                     int64_t R, const float* alpha, const float* beta, const void* v, int v_dtype, void* M,
                     int m_dtype, float* y, int64_t B, int64_t H, int64_t T, int64_t N, int64_t dv, int form,
                     void* workspace, int64_t workspace_bytes, void* stream) {
    return scan_forward_impl("sdm_scan_forward", idx_w, wt_w, W, idx_r, wt_r, R, alpha, beta, v, v_dtype, M,
                             m_dtype, y, nullptr, false, B, H, T, N, dv, form, workspace, workspace_bytes, stream);
}

int64_t sdm_scan_gated_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t W, int64_t R, int64_t dv) {
    const int64_t b = sdm_scan_workspace_bytes(B, H, T, W, R, dv);
    if (b <= 0) return b;
    return (b + 255) / 256 * 256 + B * H * T * dv * 4;  // + y, where the call keeps it itself
}

int sdm_scan_forward_gated(const int32_t* idx_w, const float* wt_w, int64_t W, const int32_t* idx_r,
                           const float* wt_r, int64_t R, const float* alpha, const float* beta, const void* v,
                           int v_dtype, void* M, int m_dtype, float* y, const float* gamma, const void* g,
                           int g_dtype, float eps, float* o, int64_t B, int64_t H, int64_t T, int64_t N,
                           int64_t dv, int form, void* workspace, int64_t workspace_bytes, void* stream) {
    const char* fn = "sdm_scan_forward_gated";
    int rc = check_scan(fn, idx_w, wt_w, W, idx_r, wt_r, R, alpha, beta, v, v_dtype, B, H, T, N, dv, form,
                        m_dtype);
    if (g_dtype != SDM_F32 && g_dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "unknown gate dtype %d", g_dtype);
    if (!(eps >= 0.f)) return fail(SDM_ERR_SHAPE, "%s: eps must be >= 0", fn);
    if (rc == NO_WORK) return ok();
    if (rc) return rc;
    if (B * H * T > 0xFFFFFFFFll)
        return fail(SDM_ERR_UNSUPPORTED, "B*H*T=%lld: at most 2^32 - 1 rows per call", (long long)(B * H * T));
    if ((rc = check_buffers(fn, {M, gamma, g, o}))) return rc;
    if (y && !aligned16(y)) return fail(SDM_ERR_ALIGN, "%s: pointer %p not 16-byte aligned", fn, (void*)y);
    if (o == y) return fail(SDM_ERR_SHAPE, "%s: o may not alias y", fn);
    const int64_t scan_ws = sdm::scan_workspace_bytes(B * H, T, (int)W, (int)R, (int)dv);
    if ((rc = check_workspace(workspace, workspace_bytes, (scan_ws + 255) / 256 * 256 + B * H * T * dv * 4)))
        return rc;
    sdm::GateArgs ga{};
    ga.gamma = gamma; ga.g = g; ga.o = o; ga.eps = eps; ga.H = H; ga.g_bf16 = g_dtype == SDM_BF16;
    const bool fused = sdm::scan_fuses_gate(B * H, T, (int)W, (int)R, (int)dv, m_dtype == SDM_BF16, form);
    // where the scan stores y itself and the caller passed none, y goes to the workspace's tail
    float* yy = y ? y : reinterpret_cast<float*>(static_cast<char*>(workspace) + (scan_ws + 255) / 256 * 256);
    sdm::ScanArgs a{};
    a.idx_w = idx_w; a.wt_w = wt_w; a.W = (int)W;
    a.idx_r = idx_r; a.wt_r = wt_r; a.R = (int)R;
    a.alpha = alpha; a.beta = beta;
    a.v = v; a.v_bf16 = v_dtype == SDM_BF16;
    a.M = M; a.m_bf16 = m_dtype == SDM_BF16;
    a.y = fused ? y : yy;
    a.NS = B * H; a.T = T; a.N = N; a.dv = (int)dv;
    a.form = form;
    a.workspace = workspace;
    a.gate = fused ? &ga : nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sdm::launch_scan(a, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (!fused) {
        sdm::OutGateArgs og{};
        og.y = yy; og.gamma = gamma; og.g = g; og.o = o; og.eps = eps;
        og.rows = B * H * T; og.T = T; og.H = H; og.dv = (int)dv; og.g_bf16 = ga.g_bf16;
        e = sdm::launch_output_gate(og, st);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    return ok();
}

}  // extern "C"

namespace {

// The scan's scratch (plan records, partial y, counters) for callers that cannot
// allocate: one array per GPU, kept until the process ends. Host code uses its
// device address from hipGetSymbolAddress, taken once per device.
constexpr int64_t SCRATCH_BYTES = 64ll << 20;
__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::once_flag g_scratch_once[MAX_DEVICES];
void* g_scratch_ptr[MAX_DEVICES];
hipError_t g_scratch_err[MAX_DEVICES];

// Device address of this GPU's scratch array (nullptr and the error on failure).
void* scratch_of(int dev, hipError_t* err) {
    std::call_once(g_scratch_once[dev], [dev] {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        g_scratch_err[dev] = e;
        g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
    });
    *err = g_scratch_err[dev];
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int sdm_scan_forward_noalloc(const int32_t* idx_w, const float* wt_w, int64_t W, const int32_t* idx_r,
                             const float* wt_r, int64_t R, const float* alpha, const float* beta, const void* v,
                             int v_dtype, void* M, int m_dtype, float* y, int64_t B, int64_t H, int64_t T,
                             int64_t N, int64_t dv, int form, void* stream) {
    const char* fn = "sdm_scan_forward_noalloc";
    int rc = check_scan(fn, idx_w, wt_w, W, idx_r, wt_r, R, alpha, beta, v, v_dtype, B, H, T, N, dv, form,
                        m_dtype);
    if (rc == NO_WORK) return ok();
    if (rc) return rc;
    if ((rc = check_buffers(fn, {M, y}))) return rc;
    const int64_t tc = sdm::scan_tokens_within(B * H, T, (int)W, (int)R, (int)dv, m_dtype == SDM_BF16, form,
                                               SCRATCH_BYTES);
    if (tc < 1)
        return fail(SDM_ERR_UNSUPPORTED,
                    "%s: B*H=%lld streams need more than the %lld-byte scratch for even one token per launch",
                    fn, (long long)(B * H), (long long)SCRATCH_BYTES);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && stream) e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (dev < 0 || dev >= MAX_DEVICES) return fail(SDM_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
    void* ws = scratch_of(dev, &e);
    if (!ws) return hip_fail(e, "sdm_scan_forward_noalloc (scratch address)");
    sdm::ScanArgs a{};
    a.idx_w = idx_w; a.wt_w = wt_w; a.W = (int)W;
    a.idx_r = idx_r; a.wt_r = wt_r; a.R = (int)R;
    a.alpha = alpha; a.beta = beta;
    a.v = v; a.v_bf16 = v_dtype == SDM_BF16;
    a.M = M; a.m_bf16 = m_dtype == SDM_BF16; a.y = y;
    a.NS = B * H; a.T = T; a.N = N; a.dv = (int)dv;
    a.form = form;
    a.workspace = ws;
    a.snap = nullptr;
    a.max_tokens = tc;
    e = sdm::launch_scan(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

int64_t sdm_scan_snapshot_bytes(int64_t B, int64_t H, int64_t T, int64_t W, int64_t dv) {
    if (B < 0 || H < 0 || T < 0 || W < 1 || dv < 1) return -1;
    return B * H * T * W * dv * 4;
}

int sdm_scan_forward_save(const int32_t* idx_w, const float* wt_w, int64_t W, const int32_t* idx_r,
                          const float* wt_r, int64_t R, const float* alpha, const float* beta, const void* v,
                          int v_dtype, float* M, float* y, float* snap, int64_t B, int64_t H, int64_t T, int64_t N,
                          int64_t dv, int form, void* workspace, int64_t workspace_bytes, void* stream) {
    return scan_forward_impl("sdm_scan_forward_save", idx_w, wt_w, W, idx_r, wt_r, R, alpha, beta, v, v_dtype, M,
                             SDM_F32, y, snap, true, B, H, T, N, dv, form, workspace, workspace_bytes, stream);
}

int64_t sdm_scan_backward_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t W, int64_t R, int64_t dv) {
    if (B < 0 || H < 0 || T < 0 || W < 1 || R < 1 || W > 256 || R > 256 || dv < 4 || dv % 4) return -1;
    if (B == 0 || H == 0 || T == 0) return 0;
    return sdm::scan_backward_workspace_bytes(B * H, T, (int)W, (int)R, (int)dv);
}

int sdm_scan_backward(const int32_t* idx_w, const float* wt_w, int64_t W, const int32_t* idx_r, const float* wt_r,
                      int64_t R, const float* alpha, const float* beta, const void* v, int v_dtype,
                      const float* snap, const float* dy, float* M, float* dM, float* dv_out, float* dalpha,
                      float* dbeta, float* dwt_w, float* dwt_r, int64_t B, int64_t H, int64_t T, int64_t N,
                      int64_t dv, int form, void* workspace, int64_t workspace_bytes, void* stream) {
    const char* fn = "sdm_scan_backward";
    int rc = check_scan(fn, idx_w, wt_w, W, idx_r, wt_r, R, alpha, beta, v, v_dtype, B, H, T, N, dv, form);
    if (rc == NO_WORK) return ok();
    if (rc) return rc;
    if (!sdm::scan_backward_geometry(B * H, (int)W, (int)R, (int)dv))
        return fail(SDM_ERR_UNSUPPORTED, "no backward kernel covers W=%lld, R=%lld, dv=%lld", (long long)W,
                    (long long)R, (long long)dv);
    if ((rc = check_buffers(fn, {snap, dy, M, dM, dv_out, dalpha, dbeta, dwt_w, dwt_r}))) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes,
                              sdm::scan_backward_workspace_bytes(B * H, T, (int)W, (int)R, (int)dv))))
        return rc;
    sdm::BwdArgs a{};
    a.idx_w = idx_w; a.wt_w = wt_w; a.W = (int)W;
    a.idx_r = idx_r; a.wt_r = wt_r; a.R = (int)R;
    a.alpha = alpha; a.beta = beta;
    a.v = v; a.v_bf16 = v_dtype == SDM_BF16;
    a.snap = snap; a.dy = dy; a.M = M; a.dM = dM;
    a.dv_out = dv_out; a.dalpha = dalpha; a.dbeta = dbeta; a.dwt_w = dwt_w; a.dwt_r = dwt_r;
    a.NS = B * H; a.T = T; a.N = N; a.dv = (int)dv;
    a.form = form;
    a.workspace = workspace;
    hipError_t e = sdm::launch_scan_backward(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

int sdm_gates(const void* x, int x_dtype, const void* W_a, const void* W_b, int w_dtype, const float* b_dt,
              const float* A, int64_t B, int64_t T, int64_t d, int64_t H, float* alpha, float* beta, void* stream) {
    const char* fn = "sdm_gates";
    if (x_dtype != SDM_F32 && x_dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "unknown x dtype %d", x_dtype);
    if (w_dtype != x_dtype) return fail(SDM_ERR_DTYPE, "weight dtype %d differs from x dtype %d", w_dtype, x_dtype);
    if (B < 0 || T < 0 || d < 1 || H < 1) return fail(SDM_ERR_SHAPE, "%s: invalid sizes", fn);
    const int64_t step = x_dtype == SDM_BF16 ? 32 : 8;
    if (d % step != 0 || d > (1 << 20))
        return fail(SDM_ERR_UNSUPPORTED, "d=%lld: a multiple of %lld up to 2^20", (long long)d, (long long)step);
    if (H > 4096) return fail(SDM_ERR_UNSUPPORTED, "H=%lld: at most 4096 heads", (long long)H);
    if (B * T > 0xFFFFFFFFll) return fail(SDM_ERR_UNSUPPORTED, "B*T=%lld: at most 2^32 - 1 tokens per call",
                                          (long long)(B * T));
    if (B == 0 || T == 0) return ok();
    int rc = check_buffers(fn, {x, W_a, W_b, b_dt, A, alpha, beta});
    if (rc) return rc;
    sdm::GatesArgs a{};
    a.x = x; a.Wa = W_a; a.Wb = W_b; a.bdt = b_dt; a.A = A; a.alpha = alpha; a.beta = beta;
    a.B = B; a.T = T; a.d = (int)d; a.H = (int)H; a.bf16 = x_dtype == SDM_BF16;
    hipError_t e = sdm::launch_gates(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

int sdm_output_gate(const float* y, const float* gamma, const void* g, int g_dtype, float eps, int64_t B,
                    int64_t H, int64_t T, int64_t dv, float* o, void* stream) {
    const char* fn = "sdm_output_gate";
    if (g_dtype != SDM_F32 && g_dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "unknown gate dtype %d", g_dtype);
    if (B < 0 || H < 1 || T < 0 || dv < 1 || !(eps >= 0.f)) return fail(SDM_ERR_SHAPE, "%s: invalid sizes or eps", fn);
    if (dv % 4 != 0) return fail(SDM_ERR_UNSUPPORTED, "dv=%lld must be a multiple of 4", (long long)dv);
    if (B * H * T > 0xFFFFFFFFll)
        return fail(SDM_ERR_UNSUPPORTED, "B*H*T=%lld: at most 2^32 - 1 rows per call", (long long)(B * H * T));
    if (B == 0 || T == 0) return ok();
    int rc = check_buffers(fn, {y, gamma, g, o});
    if (rc) return rc;
    sdm::OutGateArgs a{};
    a.y = y; a.gamma = gamma; a.g = g; a.o = o; a.eps = eps;
    a.rows = B * H * T; a.T = T; a.H = H; a.dv = (int)dv; a.g_bf16 = g_dtype == SDM_BF16;
    hipError_t e = sdm::launch_output_gate(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

int sdm_state_init_backward(const float* dM, float* dM0, int64_t B, int64_t H, int64_t N, int64_t dv,
                            void* stream) {
    if (B < 0 || H < 0 || N < 1 || dv < 1) return fail(SDM_ERR_SHAPE, "sdm_state_init_backward: invalid sizes");
    if (dv % 4 != 0) return fail(SDM_ERR_UNSUPPORTED, "sdm_state_init_backward: dv must be a multiple of 4");
    if (H == 0) return ok();
    if (B == 0) return fail(SDM_ERR_SHAPE, "sdm_state_init_backward: B must be >= 1");
    int rc = check_buffers("sdm_state_init_backward", {dM, dM0});
    if (rc) return rc;
    hipError_t e = sdm::launch_state_init_backward(dM, dM0, B, H * N * dv, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sdm_state_init_backward launch");
    return ok();
}

}  // extern "C"
